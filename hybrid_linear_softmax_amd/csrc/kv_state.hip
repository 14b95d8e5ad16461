// Linear-attention state reduction (the O(N) half of the gated linear layer:
// SANA-Video 2.0 summary page, section 03; review page, section 1):
//   S = sum_j phi(k_j) v_j^T  (d x d),   z = sum_j phi(k_j)  (d),   phi = ReLU,
// for every (batch, head).  Pass 1 gives each of C blocks of a head every C-th
// 64-token tile (block c: tiles c, c + C, c + 2C, ...) and writes one partial
// (S_c, z_c) per block; pass 2 adds the partials in block order.  No atomics:
// the result is bitwise reproducible.  With interleaved tiles the blocks of a
// head sweep its K and V together, as one front, instead of each streaming a
// region of its own: fewer concurrent DRAM streams, measured faster.
//
// bf16 pass 1 is an MFMA contraction over tokens: phi(K_c)^T V_c.  Both
// operands need "8 consecutive tokens of one feature" per lane, while K and V
// are stored token-major, so each 64-token tile is transposed on its way into
// LDS (4 tokens x 8 features per thread, in registers) and the MFMA operands
// are then plain 16-byte LDS reads.  The kernel is HBM-bound (64 flop/byte at
// d = 128), the MFMA work keeps the VALU free for the transpose.
#include "ha_device.h"
#include "ha_launch.h"

namespace ha {

namespace {

constexpr int kTile = 64;  // tokens per pass-1 tile
constexpr int64_t kSplitBlocks = 480;  // pass-1 blocks over the whole problem (at most)

// ---------------------------------------------------------------- bf16 pass 1
// wz (optional, [B*H, N] float32) weights the z sum: z = sum_j wz_j phi(k_j)
// (the backward pass's dz = sum_i dden_i phi(q_i)); null gives the plain sum.
template <int D>
__global__ __launch_bounds__(256) void kv_partials_bf16(const bf16_t* __restrict__ K,
                                                        const bf16_t* __restrict__ V,
                                                        float* __restrict__ part, int64_t N,
                                                        int64_t chunks, const float* __restrict__ wz) {
  constexpr int P = kTile + 8;            // LDS pitch (elements) of a transposed row
  constexpr int FG = D / 8;               // 16-byte feature groups per token row
  constexpr int SUB = (kTile / 4) * FG;   // 4-token x 8-feature sub-tiles per tensor
  constexpr int PER = 2 * SUB / 256;      // sub-tiles per thread (K and V together)
  constexpr int RB = D / 64;              // 32x32 output blocks per wave, per dim
  __shared__ __attribute__((aligned(16))) bf16_t sK[D * P];  // phi(K)^T tile [feature][token]
  __shared__ __attribute__((aligned(16))) bf16_t sV[D * P];  // V^T tile      [feature][token]
  __shared__ float sZ[kTile / 4][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t bh = blockIdx.x / chunks;
  const int64_t c = blockIdx.x % chunks;
  const int64_t t_begin = c * kTile;        // first token of this block's first tile
  const int64_t t_step = chunks * kTile;    // tokens between this block's tiles
  const bf16_t* Kh = K + bh * N * D;
  const bf16_t* Vh = V + bh * N * D;

  // sub-tile u of this thread: tensor u / SUB, feature group, 4-token group.
  // The token group is the fast index across lanes: the transposed 8-byte LDS
  // stores of 16 consecutive lanes then fill one 128-byte row segment (distinct
  // banks), while each 64-byte piece of a token row is still read by 4 lanes.
  int sub_fg[PER], sub_m[PER];
  bool sub_k[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int u = tid + 256 * i;
    sub_k[i] = u < SUB;
    const int w = u % SUB;
    sub_fg[i] = w / (kTile / 4);
    sub_m[i] = w % (kTile / 4);
  }

  uint4 regs[PER][4];
  auto load_tile = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bf16_t* src = sub_k[i] ? Kh : Vh;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tok = t0 + 4 * sub_m[i] + r;
        regs[i][r] = tok < N ? *reinterpret_cast<const uint4*>(src + tok * D + 8 * sub_fg[i])
                             : make_uint4(0, 0, 0, 0);
      }
    }
  };

  float zacc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) zacc[k] = 0.f;

  f32x16 acc[RB][RB];
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // wave's output block: rows (key features) ra.., cols (value features) cj..
  const int ra = (wave >> 1) * 32 * RB;
  const int cj = (wave & 1) * 32 * RB;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  load_tile(t_begin);
  for (int64_t t0 = t_begin; t0 < N; t0 += t_step) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      uint4 w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = sub_k[i] ? relu8(regs[i][r]) : regs[i][r];
      if (sub_k[i]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (wz == nullptr) {
            zacc[0] += bf_lo(w[r].x); zacc[1] += bf_hi(w[r].x);
            zacc[2] += bf_lo(w[r].y); zacc[3] += bf_hi(w[r].y);
            zacc[4] += bf_lo(w[r].z); zacc[5] += bf_hi(w[r].z);
            zacc[6] += bf_lo(w[r].w); zacc[7] += bf_hi(w[r].w);
          } else {
            const int64_t tok = t0 + 4 * sub_m[i] + r;
            const float wt = tok < N ? wz[bh * N + tok] : 0.f;
            zacc[0] = fmaf(wt, bf_lo(w[r].x), zacc[0]); zacc[1] = fmaf(wt, bf_hi(w[r].x), zacc[1]);
            zacc[2] = fmaf(wt, bf_lo(w[r].y), zacc[2]); zacc[3] = fmaf(wt, bf_hi(w[r].y), zacc[3]);
            zacc[4] = fmaf(wt, bf_lo(w[r].z), zacc[4]); zacc[5] = fmaf(wt, bf_hi(w[r].z), zacc[5]);
            zacc[6] = fmaf(wt, bf_lo(w[r].w), zacc[6]); zacc[7] = fmaf(wt, bf_hi(w[r].w), zacc[7]);
          }
        }
      }
      uint2 tr[8];
      transpose4x8(w, tr);
      bf16_t* dst = sub_k[i] ? sK : sV;
#pragma unroll
      for (int f = 0; f < 8; ++f)
        *reinterpret_cast<uint2*>(dst + (8 * sub_fg[i] + f) * P + 4 * sub_m[i]) = tr[f];
    }
    __syncthreads();
    if (t0 + t_step < N) load_tile(t0 + t_step);
#pragma unroll
    for (int s = 0; s < kTile / 16; ++s) {
      bf16x8 af[RB], bfr[RB];
#pragma unroll
      for (int a = 0; a < RB; ++a)
        af[a] = *reinterpret_cast<const bf16x8*>(sK + (ra + 32 * a + l32) * P + 16 * s + 8 * h);
#pragma unroll
      for (int b = 0; b < RB; ++b)
        bfr[b] = *reinterpret_cast<const bf16x8*>(sV + (cj + 32 * b + l32) * P + 16 * s + 8 * h);
#pragma unroll
      for (int a = 0; a < RB; ++a)
#pragma unroll
        for (int b = 0; b < RB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
  }

  float* out = part + (bh * chunks + c) * (int64_t)(D * D + D);
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = ra + 32 * a + 8 * (r >> 2) + 4 * h + (r & 3);
        const int col = cj + 32 * b + l32;
        out[row * D + col] = acc[a][b][r];
      }

  // z: the thread holding K sub-tile (fg, m) summed 8 features over its tokens;
  // add the 16 token groups of each feature in a fixed order.
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (sub_k[i])
#pragma unroll
      for (int k = 0; k < 8; ++k) sZ[sub_m[i]][8 * sub_fg[i] + k] = zacc[k];
  __syncthreads();
  if (tid < D) {
    float zs = 0.f;
#pragma unroll
    for (int m = 0; m < kTile / 4; ++m) zs += sZ[m][tid];
    out[D * D + tid] = zs;
  }
}

// ---------------------------------------------------------------- f32 pass 1
// Plain VALU contraction: thread (ta, tj) owns S rows ta + 16x, columns tj + 16y.
template <int D>
__global__ __launch_bounds__(256) void kv_partials_f32(const float* __restrict__ K,
                                                       const float* __restrict__ V,
                                                       float* __restrict__ part, int64_t N,
                                                       int64_t chunks, const float* __restrict__ wz) {
  constexpr int T = 32;
  constexpr int R = D / 16;
  __shared__ __attribute__((aligned(16))) float sK[T][D];
  __shared__ __attribute__((aligned(16))) float sV[T][D];
  const int tid = threadIdx.x;
  const int ta = tid >> 4, tj = tid & 15;
  const int64_t bh = blockIdx.x / chunks;
  const int64_t c = blockIdx.x % chunks;
  const int64_t t_begin = c * T;          // block c: 32-token tiles c, c + C, ...
  const int64_t t_step = chunks * T;
  const float* Kh = K + bh * N * D;
  const float* Vh = V + bh * N * D;

  float acc[R][R];
  float zacc[R];
#pragma unroll
  for (int x = 0; x < R; ++x) {
    zacc[x] = 0.f;
#pragma unroll
    for (int y = 0; y < R; ++y) acc[x][y] = 0.f;
  }
  __shared__ float sW[T];
  for (int64_t t0 = t_begin; t0 < N; t0 += t_step) {
    __syncthreads();
    if (tid < T) sW[tid] = (t0 + tid < N) ? (wz == nullptr ? 1.f : wz[bh * N + t0 + tid]) : 0.f;
    for (int e = tid; e < T * D / 4; e += 256) {
      const int row = e / (D / 4), col = 4 * (e % (D / 4));
      const int64_t tok = t0 + row;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (tok < N) {
        kv = *reinterpret_cast<const float4*>(Kh + tok * D + col);
        vv = *reinterpret_cast<const float4*>(Vh + tok * D + col);
      }
      kv.x = fmaxf(kv.x, 0.f); kv.y = fmaxf(kv.y, 0.f);
      kv.z = fmaxf(kv.z, 0.f); kv.w = fmaxf(kv.w, 0.f);
      *reinterpret_cast<float4*>(&sK[row][col]) = kv;
      *reinterpret_cast<float4*>(&sV[row][col]) = vv;
    }
    __syncthreads();
    for (int n = 0; n < T; ++n) {
      float kr[R], vr[R];
#pragma unroll
      for (int x = 0; x < R; ++x) kr[x] = sK[n][ta + 16 * x];
#pragma unroll
      for (int y = 0; y < R; ++y) vr[y] = sV[n][tj + 16 * y];
      const float wt = sW[n];
#pragma unroll
      for (int x = 0; x < R; ++x) {
        zacc[x] = fmaf(wt, kr[x], zacc[x]);
#pragma unroll
        for (int y = 0; y < R; ++y) acc[x][y] = fmaf(kr[x], vr[y], acc[x][y]);
      }
    }
  }
  float* out = part + (bh * chunks + c) * (int64_t)(D * D + D);
#pragma unroll
  for (int x = 0; x < R; ++x)
#pragma unroll
    for (int y = 0; y < R; ++y) out[(ta + 16 * x) * D + tj + 16 * y] = acc[x][y];
  if (tj == 0)
#pragma unroll
    for (int x = 0; x < R; ++x) out[D * D + ta + 16 * x] = zacc[x];
}

// ---------------------------------------------------------------- pass 2
// Element e of (S, z) of one head: sum over chunks in order.  The bf16 path also
// stores S^T split into bf16 hi + lo (hi = rne(s), lo = rne(s - hi)), the layout
// the apply kernel's MFMA B operand reads.
// S_hi / S_lo (optional) receive the same split untransposed ([a][j]), the
// layout the backward pass's products with S^T read.
template <int D>
__global__ __launch_bounds__(256) void kv_reduce(const float* __restrict__ part,
                                                 float* __restrict__ S, float* __restrict__ z,
                                                 bf16_t* __restrict__ St_hi,
                                                 bf16_t* __restrict__ St_lo, int64_t chunks,
                                                 int blocks_per_head, bf16_t* __restrict__ S_hi,
                                                 bf16_t* __restrict__ S_lo) {
  constexpr int E = D * D + D;
  const int64_t bh = blockIdx.x / blocks_per_head;
  const int e = (blockIdx.x % blocks_per_head) * 256 + threadIdx.x;
  if (e >= E) return;
  const float* p = part + bh * chunks * (int64_t)E + e;
  float s = 0.f;
  for (int64_t c = 0; c < chunks; ++c) s += p[c * E];
  if (e < D * D) {
    S[bh * D * D + e] = s;
    if (St_hi != nullptr) {
      const int a = e / D, j = e % D;
      const bf16_t hi = to_bf16(s);
      const float hif = __uint_as_float(static_cast<uint32_t>(hi) << 16);
      const bf16_t lo = to_bf16(s - hif);
      St_hi[bh * D * D + j * D + a] = hi;
      St_lo[bh * D * D + j * D + a] = lo;
      if (S_hi != nullptr) {
        S_hi[bh * D * D + e] = hi;
        S_lo[bh * D * D + e] = lo;
      }
    }
  } else {
    z[bh * D + (e - D * D)] = s;
  }
}

}  // namespace

KvSplit kv_split(int64_t BH, int64_t N) {
  // Blocks per head: floor(kSplitBlocks / BH), so that the whole grid stays
  // within one wave of resident blocks (two per CU; past 512 blocks the excess
  // runs as a tail: 720p/5s 169 -> 226 us at 528 blocks), at least one, at most
  // one per 64-token tile.  A function of (B*H, N) only, never of the device:
  // the split fixes the order of the reduction and therefore the result.
  if (N <= 0) return KvSplit{0};
  int64_t per_head = BH > 0 ? kSplitBlocks / BH : 1;
  if (per_head < 1) per_head = 1;
  const int64_t tiles = (N + kTile - 1) / kTile;
  return KvSplit{per_head < tiles ? per_head : tiles};
}

hipError_t launch_kv_partials(bool bf16, int d, const void* K, const void* V, float* part,
                              int64_t BH, int64_t N, KvSplit sp, hipStream_t s, const float* wz) {
  if (sp.chunks == 0 || BH == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(BH * sp.chunks)), block(256);
  if (bf16) {
    const bf16_t* k = static_cast<const bf16_t*>(K);
    const bf16_t* v = static_cast<const bf16_t*>(V);
    if (d == 128)
      kv_partials_bf16<128><<<grid, block, 0, s>>>(k, v, part, N, sp.chunks, wz);
    else
      kv_partials_bf16<64><<<grid, block, 0, s>>>(k, v, part, N, sp.chunks, wz);
  } else {
    const float* k = static_cast<const float*>(K);
    const float* v = static_cast<const float*>(V);
    if (d == 128)
      kv_partials_f32<128><<<grid, block, 0, s>>>(k, v, part, N, sp.chunks, wz);
    else
      kv_partials_f32<64><<<grid, block, 0, s>>>(k, v, part, N, sp.chunks, wz);
  }
  return hipGetLastError();
}

hipError_t launch_kv_reduce(bool bf16, int d, const float* part, float* S, float* z,
                            uint16_t* St_hi, uint16_t* St_lo, int64_t BH, int64_t chunks,
                            hipStream_t s, uint16_t* S_hi, uint16_t* S_lo) {
  if (BH == 0) return hipSuccess;
  const int E = d * d + d;
  const int bph = (E + 255) / 256;
  const dim3 grid(static_cast<unsigned>(BH * bph)), block(256);
  bf16_t* hi = bf16 ? St_hi : nullptr;
  bf16_t* lo = bf16 ? St_lo : nullptr;
  bf16_t* shi = bf16 && St_hi != nullptr ? S_hi : nullptr;
  bf16_t* slo = bf16 && St_hi != nullptr ? S_lo : nullptr;
  if (d == 128)
    kv_reduce<128><<<grid, block, 0, s>>>(part, S, z, hi, lo, chunks, bph, shi, slo);
  else
    kv_reduce<64><<<grid, block, 0, s>>>(part, S, z, hi, lo, chunks, bph, shi, slo);
  return hipGetLastError();
}

}  // namespace ha
