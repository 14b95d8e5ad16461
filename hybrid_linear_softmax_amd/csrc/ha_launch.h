// Host-side launchers of the gfx950 kernels (internal to libhybrid_attn.so).
// Each returns the hipError_t of its launch(es); shapes are validated by the
// C-ABI layer before any of these is called.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace ha {

// Token split of the linear-state reduction: a pure function of (BH, N), never
// of the device, so the reduction order (and the result) is reproducible.
struct KvSplit {
  int64_t chunks;     // pass-1 blocks (partials) per head; block c takes every
                      // chunks-th tile starting at tile c; 0 when N == 0
};
KvSplit kv_split(int64_t BH, int64_t N);

// Workspace layout of the linear layer (byte offsets from the workspace base).
struct LinearWs {
  size_t part;    // float [BH][chunks][d*d + d]  per-chunk partial S, z
  size_t S;       // float [BH][d][d]             reduced S (row = key feature)
  size_t z;       // float [BH][d]                reduced z
  size_t St_hi;   // bf16  [BH][d][d]             S^T split hi (bf16 path only)
  size_t St_lo;   // bf16  [BH][d][d]             S^T - hi, rounded (bf16 path only)
  size_t total;
};
LinearWs linear_ws(int64_t BH, int64_t N, int d, bool bf16);

// R1 pass 1: per (bh, chunk) partial state into part.
// wz (optional, [BH, N] float32) weights the z sum per token.
hipError_t launch_kv_partials(bool bf16, int d, const void* K, const void* V, float* part,
                              int64_t BH, int64_t N, KvSplit split, hipStream_t s,
                              const float* wz = nullptr);
// R1 pass 2: fixed-order sum over chunks into S, z (and the bf16 hi/lo S^T).
// S_hi/S_lo (optional, bf16 path) also receive the untransposed hi/lo split.
hipError_t launch_kv_reduce(bool bf16, int d, const float* part, float* S, float* z,
                            uint16_t* St_hi, uint16_t* St_lo, int64_t BH, int64_t chunks,
                            hipStream_t s, uint16_t* S_hi = nullptr, uint16_t* S_lo = nullptr);
// R2: fused apply phi(Q) S / (phi(Q) z + eps), sigmoid gate, store.
hipError_t launch_apply(bool bf16, int d, const void* Q, const void* G, void* O, const float* S,
                        const float* z, const uint16_t* St_hi, const uint16_t* St_lo, int64_t BH,
                        int64_t N, float eps, hipStream_t s);
// Query / key block sizes of the block-sparse anchor's pattern.
constexpr int kSparseBlockQ = 256;
constexpr int kSparseBlockK = 64;
// R3: gated softmax anchor (flash-style, online softmax).  With blk_off set,
// block-sparse: query block qb (kSparseBlockQ rows) attends to the key blocks
// (kSparseBlockK keys) blk_idx[blk_off[qb] .. blk_off[qb+1]-1], n_idx entries.
hipError_t launch_anchor(bool bf16, int d, const void* Q, const void* K, const void* V,
                         const void* G, void* O, int64_t BH, int64_t N, hipStream_t s,
                         const int32_t* blk_off = nullptr, const int32_t* blk_idx = nullptr,
                         int64_t n_idx = 0, float* lse = nullptr);
// Backward pass of the anchor given O, dO and the forward's lse (see anchor_bwd.hip).
size_t softmax_bwd_ws(int64_t BH, int64_t N, int d, bool bf16);
hipError_t launch_softmax_backward(bool bf16, int d, const void* Q, const void* K, const void* V,
                                   const void* G, const void* O, const void* dO, const float* lse,
                                   void* dQ, void* dK, void* dV, void* dG, int64_t BH, int64_t N,
                                   void* ws, hipStream_t s);

// Workspace of the linear layer's backward pass (byte offsets).
struct LinearBwdWs {
  size_t part;                    // float [BH][chunks][d*d + d], reused by both reductions
  size_t S, z, dS, dz;            // float [BH][d][d], [BH][d]
  size_t St_hi, St_lo, S_hi, S_lo;      // bf16 [BH][d][d] (bf16 path only)
  size_t dSt_hi, dSt_lo, dS_hi, dS_lo;  // bf16 [BH][d][d] (bf16 path only)
  size_t dn;                      // [BH][N][d] in the I/O dtype
  size_t dden;                    // float [BH][N]
  size_t total;
};
LinearBwdWs linear_bwd_ws(int64_t BH, int64_t N, int d, bool bf16);
// dQ, dK, dV, dG of the gated linear layer given dO (six passes, see linear_bwd.hip).
hipError_t launch_linear_backward(bool bf16, int d, const void* Q, const void* K, const void* V,
                                  const void* G, const void* dO, void* dQ, void* dK, void* dV, void* dG,
                                  int64_t BH, int64_t N, float eps, void* ws, hipStream_t s);

// AttnRes mixture over candidates summaries[0 .. M-1] then x (each [tokens, C]).
int attnres_max_candidates();
hipError_t launch_attnres_mix(bool bf16, const void* summaries, int M, const void* x, const float* w, void* h,
                              int64_t tokens, int C, float eps, hipStream_t s);

// Block projections: Q, K, V, G = split_heads(x W_in^T) and
// x_out = x + concat_heads(O) W_out^T (x_out may be x).
hipError_t launch_proj_in(bool bf16, const void* x, const void* W_in, void* Q, void* K, void* V, void* G,
                          int64_t B, int64_t H, int64_t N, int d, hipStream_t s);
hipError_t launch_proj_out(bool bf16, const void* O, const void* W_out, const void* x, void* x_out,
                           int64_t B, int64_t H, int64_t N, int d, hipStream_t s);

// Achievable-peak probes (see probe.hip).
double probe_mfma_flops(int blocks, int iters);
hipError_t launch_probe_mfma(int blocks, int iters, float* sink, hipStream_t s);
hipError_t launch_probe_mfma_data(int blocks, int iters, float* sink, hipStream_t s);
hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, bool nontemporal, hipStream_t s);
hipError_t launch_probe_overlap(int mode, int waves_per_simd, int blocks, int iters, float* sink, hipStream_t s);

}  // namespace ha
