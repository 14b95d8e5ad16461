// Fused apply of the gated linear layer (SANA-Video 2.0 summary page, section
// 03; review page, section 1):
//   o_i = sigmoid(g_i) * (phi(q_i)^T S) / (phi(q_i) . z + eps)
// streaming Q and G in and O out once.  At d = 128 this is 2 d^2 flops per
// 6 d bytes, more than the VALU can sustain at HBM speed, so phi(Q) S runs on
// bf16 MFMA.  S is held as an unevaluated bf16 pair S^T = hi + lo (both halves
// rounded to nearest even), so the product carries ~16 significant bits of S
// while phi(q) -- the bf16 input itself -- is exact.  Each wave keeps its
// quarter of S^T (hi and lo) in registers for the whole kernel.  The blocks of
// a head take its 64-token tiles interleaved (block b: tiles b, b + B_h, ...),
// so that they stream Q, G and O as one front per head rather than each a
// region of its own (fewer concurrent DRAM streams, measured faster).
#include "ha_device.h"
#include "ha_launch.h"

namespace ha {

namespace {

constexpr int kTok = 64;  // tokens per tile
constexpr int64_t kApplyBlocksPerHead = 64;  // bf16 apply blocks per (b, h)

template <int D>
__global__ __launch_bounds__(256) void apply_bf16(const bf16_t* __restrict__ Q,
                                                  const bf16_t* __restrict__ G,
                                                  bf16_t* __restrict__ O,
                                                  const bf16_t* __restrict__ St_hi,
                                                  const bf16_t* __restrict__ St_lo,
                                                  const float* __restrict__ z, int64_t N,
                                                  int64_t blocks_per_head, float eps) {
  constexpr int QP = D + 8;            // LDS pitch of the phi(Q) tile (elements)
  constexpr int NP = D + 4;            // LDS pitch of the numerator tile (floats)
  constexpr int FG = D / 8;            // 16-byte groups per token row
  constexpr int CH = kTok * FG / 256;  // 16-byte chunks per thread per tile
  constexpr int NB = D / 64;           // 16-column MFMA blocks per wave
  constexpr int KS = D / 32;           // k-steps of the 16x16x32 MFMA
  __shared__ __attribute__((aligned(16))) bf16_t sQ[kTok * QP];
  __shared__ __attribute__((aligned(16))) float sNum[kTok * NP];
  __shared__ float sDen[kTok];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int kq = lane >> 4;
  const int64_t bh = blockIdx.x / blocks_per_head;
  const int64_t blk = blockIdx.x % blocks_per_head;
  const int64_t base = bh * N * D;

  // B operand: S^T rows j = this wave's output columns, k = key features.
  bf16x8 bhi[NB][KS], blo[NB][KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int j = wave * (D / 4) + 16 * nb + c16;
      const int64_t off = bh * D * D + j * D + 32 * s + 8 * kq;
      bhi[nb][s] = as_bf16x8(*reinterpret_cast<const uint4*>(St_hi + off));
      blo[nb][s] = as_bf16x8(*reinterpret_cast<const uint4*>(St_lo + off));
    }
  const int fg = tid % FG;  // the feature group of every chunk of this thread
  float zf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) zf[k] = z[bh * D + 8 * fg + k];

  const int64_t ntiles = (N + kTok - 1) / kTok;
  const int64_t tb = blk;               // this block's tiles: tb, tb + ts, ...
  const int64_t ts = blocks_per_head;

  // Q and G chunks of one tile: chunk c = tid + 256 i -> token c / FG, features
  // 8 (c % FG) .. + 7 (the feature group is the same for every chunk of a thread)
  uint4 qv[CH], gv[CH];
  auto load_tile = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t tok = t * kTok + (tid + 256 * i) / FG;
      qv[i] = make_uint4(0, 0, 0, 0);
      gv[i] = make_uint4(0, 0, 0, 0);
      if (t < ntiles && tok < N) {
        qv[i] = load_stream(Q + base + tok * D + 8 * fg);
        gv[i] = load_stream(G + base + tok * D + 8 * fg);
      }
    }
  };
  load_tile(tb);
  for (int64_t t = tb; t < ntiles; t += ts) {
    const int64_t tok0 = t * kTok;
    uint4 gcur[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int row = (tid + 256 * i) / FG;
      const uint4 q = relu8(qv[i]);
      gcur[i] = gv[i];
      float dp = bf_lo(q.x) * zf[0];
      dp = fmaf(bf_hi(q.x), zf[1], dp);
      dp = fmaf(bf_lo(q.y), zf[2], dp);
      dp = fmaf(bf_hi(q.y), zf[3], dp);
      dp = fmaf(bf_lo(q.z), zf[4], dp);
      dp = fmaf(bf_hi(q.z), zf[5], dp);
      dp = fmaf(bf_lo(q.w), zf[6], dp);
      dp = fmaf(bf_hi(q.w), zf[7], dp);
#pragma unroll
      for (int m = 1; m < FG; m <<= 1) dp += __shfl_xor(dp, m);
      *reinterpret_cast<uint4*>(sQ + row * QP + 8 * fg) = q;
      if (fg == 0) sDen[row] = dp + eps;
    }
    __syncthreads();
    load_tile(t + ts);  // next tile's Q and G stream in during this tile's MFMAs
#pragma unroll
    for (int mb = 0; mb < kTok / 16; ++mb) {
      f32x4 acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(sQ + (16 * mb + c16) * QP + 32 * s + 8 * kq);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhi[nb][s], acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, blo[nb][s], acc[nb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sNum[(16 * mb + 4 * kq + r) * NP + wave * (D / 4) + 16 * nb + c16] = acc[nb][r];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int row = (tid + 256 * i) / FG;
      const int64_t tok = tok0 + row;
      if (tok < N) {
        const float4 n0 = *reinterpret_cast<const float4*>(sNum + row * NP + 8 * fg);
        const float4 n1 = *reinterpret_cast<const float4*>(sNum + row * NP + 8 * fg + 4);
        const float inv = __builtin_amdgcn_rcpf(sDen[row]);
        const uint4 g = gcur[i];
        uint4 o;
        o.x = pack_bf16(gate_fast(bf_lo(g.x)) * n0.x * inv, gate_fast(bf_hi(g.x)) * n0.y * inv);
        o.y = pack_bf16(gate_fast(bf_lo(g.y)) * n0.z * inv, gate_fast(bf_hi(g.y)) * n0.w * inv);
        o.z = pack_bf16(gate_fast(bf_lo(g.z)) * n1.x * inv, gate_fast(bf_hi(g.z)) * n1.y * inv);
        o.w = pack_bf16(gate_fast(bf_lo(g.w)) * n1.z * inv, gate_fast(bf_hi(g.w)) * n1.w * inv);
        store_stream(O + base + tok * D + 8 * fg, o);
      }
    }
    __syncthreads();
  }
}

// Plain float32 apply: phi(Q) tile in LDS, S and z read through the caches,
// thread (token, column slice).
template <int D>
__global__ __launch_bounds__(256) void apply_f32(const float* __restrict__ Q,
                                                 const float* __restrict__ G,
                                                 float* __restrict__ O, const float* __restrict__ S,
                                                 const float* __restrict__ z, int64_t N,
                                                 int64_t tiles_per_block, int64_t blocks_per_head,
                                                 float eps) {
  constexpr int T = 16;
  __shared__ float sQ[T * D];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / blocks_per_head;
  const int64_t blk = blockIdx.x % blocks_per_head;
  const int64_t base = bh * N * D;
  const float* Sh = S + bh * D * D;
  const float* zh = z + bh * D;
  const int row = tid >> 4, tj = tid & 15;
  const int64_t ntiles = (N + T - 1) / T;
  const int64_t tb = blk * tiles_per_block;
  const int64_t te = min(ntiles, tb + tiles_per_block);
  for (int64_t t = tb; t < te; ++t) {
    const int64_t tok0 = t * T;
    __syncthreads();
    for (int e = tid; e < T * D; e += 256) {
      const int64_t tok = tok0 + e / D;
      sQ[e] = tok < N ? fmaxf(Q[base + tok * D + e % D], 0.f) : 0.f;
    }
    __syncthreads();
    const int64_t tok = tok0 + row;
    if (tok < N) {
      float den = 0.f;
      for (int a = 0; a < D; ++a) den = fmaf(sQ[row * D + a], zh[a], den);
      den += eps;
      for (int y = 0; y < D / 16; ++y) {
        const int j = tj + 16 * y;
        float num = 0.f;
        for (int a = 0; a < D; ++a) num = fmaf(sQ[row * D + a], Sh[a * D + j], num);
        const int64_t off = base + tok * D + j;
        O[off] = gate_exact(G[off]) * (num / den);
      }
    }
  }
}

// Blocks per head of the bf16 apply: kApplyBlocksPerHead (each taking every
// kApplyBlocksPerHead-th tile of its head), at most one per tile.  Measured
// within 0.2 % of the best grid at 480p, 720p/5s, 14B and 14B B=2.
int64_t apply_blocks_per_head(int64_t ntiles) {
  return kApplyBlocksPerHead < ntiles ? kApplyBlocksPerHead : ntiles;
}

}  // namespace

hipError_t launch_apply(bool bf16, int d, const void* Q, const void* G, void* O, const float* S,
                        const float* z, const uint16_t* St_hi, const uint16_t* St_lo, int64_t BH,
                        int64_t N, float eps, hipStream_t s) {
  if (BH == 0 || N == 0) return hipSuccess;
  const int tile = bf16 ? kTok : 16;
  const int64_t ntiles = (N + tile - 1) / tile;
  if (bf16) {
    // blocks per head from the measured grid rule (the apply has no cross-block
    // reduction: the grid does not affect the result)
    const int64_t bph = apply_blocks_per_head(ntiles);
    const dim3 grid(static_cast<unsigned>(BH * bph)), block(256);
    const bf16_t* q = static_cast<const bf16_t*>(Q);
    const bf16_t* g = static_cast<const bf16_t*>(G);
    bf16_t* o = static_cast<bf16_t*>(O);
    if (d == 128)
      apply_bf16<128><<<grid, block, 0, s>>>(q, g, o, St_hi, St_lo, z, N, bph, eps);
    else
      apply_bf16<64><<<grid, block, 0, s>>>(q, g, o, St_hi, St_lo, z, N, bph, eps);
  } else {
    // about 2048 blocks, each walking a contiguous run of tiles of one head
    int64_t bph = (2048 + BH - 1) / BH;
    if (bph > ntiles) bph = ntiles;
    const int64_t tpb = (ntiles + bph - 1) / bph;
    bph = (ntiles + tpb - 1) / tpb;
    const dim3 grid(static_cast<unsigned>(BH * bph)), block(256);
    const float* q = static_cast<const float*>(Q);
    const float* g = static_cast<const float*>(G);
    float* o = static_cast<float*>(O);
    if (d == 128)
      apply_f32<128><<<grid, block, 0, s>>>(q, g, o, S, z, N, tpb, bph, eps);
    else
      apply_f32<64><<<grid, block, 0, s>>>(q, g, o, S, z, N, tpb, bph, eps);
  }
  return hipGetLastError();
}

}  // namespace ha
