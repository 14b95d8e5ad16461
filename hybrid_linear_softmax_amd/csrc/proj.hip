// Projections of the attention block around the hybrid group (SANA-Video 2.0
// review page, section 3: the hybrid attention inside the DiT blocks of the
// compiled forward; summary page, section 03):
//   proj_in:  [Q | K | V | G] = x W_in^T, x: [B, N, C], W_in: [4C, C], each
//             C-wide block split into H heads of d features -> [B, H, N, d];
//   proj_out: x_out = x + concat_h(O) W_out^T, O: [B, H, N, d], W_out: [C, C].
// Both are dense contractions over C, run on the bf16 MFMA with float32
// accumulation.
//
// bf16 kernel: one block = 256 output features x 256 tokens, 8 waves, each
// owning 128 features x 64 tokens of the output, K in steps of 32.
//  * the product is taken transposed, out^T = W x^T: the MFMA A operand is a
//    weight row, the B operand a token row, both contiguous along C, and a
//    lane's accumulator holds four consecutive output features of one token --
//    an 8-byte store in either epilogue (the head scatter of proj_in, the
//    residual add of proj_out);
//  * two-group ping-pong: waves 0-3 and 4-7 (one of each per SIMD) alternate,
//    between block barriers, a compute phase -- 16 MFMAs on operands already in
//    registers -- and a memory phase -- the LDS reads of the operands of their
//    next K step and the loads of a K step three ahead -- so that in every phase
//    one wave per SIMD keeps the matrix core busy.  Each group runs a loop of its
//    own (phases in opposite order), with no role branch inside it;
//  * K tiles come straight from global memory into LDS (buffer loads to LDS, 16
//    bytes per lane, no registers): a ring of four 32 KB stages, rows of 64 bytes
//    whose 16-byte chunks are XOR-swizzled by row so that the fragment reads of
//    32 consecutive rows hit distinct banks; group 0 loads the weight half of a
//    stage, group 1 the token half.  A lane's offset is fixed for the kernel and
//    the K step is the scalar offset, the wave index sits in a scalar register
//    and the loops are unrolled by the ring's depth, so neither the loads nor the
//    fragment reads need per-lane address arithmetic (on this part vector
//    instructions of one wave do not issue under another wave's MFMAs).  Waits
//    on those loads are explicit (the compiler does not track them), placed
//    before the barrier that precedes a stage's first read;
//  * proj_out reads its token rows straight out of O's [B, H, N, d] layout: a
//    32-wide K step lies inside one head, so a row is 64 contiguous bytes;
//  * tiles past M tokens or the last feature clamp their load rows to the last
//    valid row (valid memory, results never stored), so no load is predicated;
//  * tiles are ordered in groups of 4 token tiles x all feature tiles and the
//    order is split into 8 contiguous ranges, one per XCD, so the blocks that
//    run together on one XCD share token rows and weight rows in its L2.
#include <type_traits>

#include "ha_device.h"
#include "ha_launch.h"

namespace ha {

namespace {

constexpr int kTF = 256;   // output features per block
constexpr int kTM = 256;   // tokens per block
constexpr int kTK = 32;    // K per step
constexpr int kGroupM = 4; // token tiles per ordering group
constexpr int kStages = 4; // LDS ring
constexpr int kStage = (kTF + kTM) * kTK;  // elements per stage: weight rows, then token rows

// chunk swizzle of a stage row: 16-byte chunk c of row r sits in slot c ^ swz(r).
// Rows are 64 bytes, so rows r and r + 4 fall on the same LDS banks; the slot
// has to change with r >> 2.  Measured with ds_read_b128 of 32 consecutive rows
// per half-wave: (r ^ (r >> 2)) & 3 reads at the speed of a conflict-free
// pattern, while ((r >> 1) ^ (r >> 3)) & 3 took 1.6x as long.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 2)) & 3; }

// s_waitcnt vmcnt(n) with the LDS and export counters left at their maxima
#define HA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// 16 bytes per lane from global memory straight into LDS at dst + 16 lane (dst
// wave-uniform).  Kept out of the kernel's lambdas: a target builtin inside a
// lambda can make the host compilation drop the kernel's launch stub.
__device__ __forceinline__ void global_to_lds16(const bf16_t* src, bf16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// The same through a buffer descriptor: byte address base + voff (per lane,
// fixed for the kernel) + soff (wave-uniform, the K step): no vector
// instruction per load.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, bf16_t* dst, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, static_cast<int>(voff), soff, 0, 0);
}

// block barrier after this wave's LDS accesses have completed; the sched and
// asm barriers keep the phases' instructions on their side of it
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

struct ProjShape {
  int64_t M;      // tokens B * N
  int64_t Nf;     // output features (4C or C)
  int64_t K;      // C
  int64_t N;      // tokens per batch item
  int64_t H;
  int d;
  int lgd;        // log2(d): d is 64 or 128
  int64_t nt_f, nt_m, total;
};

__device__ __forceinline__ void tile_of(int64_t t, const ProjShape& p, int64_t& tf, int64_t& tm) {
  const int64_t g = t / (kGroupM * p.nt_f);
  const int64_t gm = min((int64_t)kGroupM, p.nt_m - g * kGroupM);
  const int64_t idx = t - g * kGroupM * p.nt_f;
  tf = idx / gm;
  tm = g * kGroupM + idx % gm;
}

// MODE 0: proj_in, X = x [M, K], outputs scattered into out[0..3] = Q, K, V, G.
// MODE 1: proj_out, X = O [B, H, N, d] read as [M, K], out[0] = resid + X W^T;
// out0 may be resid itself (each element is read, then written, by one lane).
// WIDE (proj_out only): O spans 4 GB or more, beyond 32-bit buffer offsets from
// its start; its token rows are then loaded through 64-bit lane addresses.
template <int MODE, bool WIDE>
__global__ __launch_bounds__(512, 1) void proj_bf16(const bf16_t* __restrict__ X,
                                                    const bf16_t* __restrict__ W,
                                                    bf16_t* out0, bf16_t* __restrict__ out1,
                                                    bf16_t* __restrict__ out2, bf16_t* __restrict__ out3,
                                                    const bf16_t* resid, ProjShape p) {
  __shared__ __attribute__((aligned(1024))) bf16_t lds[kStages * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index, and all that derives from it, in scalar registers: load
  // destinations and descriptors need no per-lane arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int wf = wave >> 2;  // group: 128-feature half, and the half of each stage it loads
  const int wt = wave & 3;   // 64-token quarter
  int64_t tf, tm;
  tile_of(xcd_remap(blockIdx.x, p.total), p, tf, tm);
  const int64_t f0 = tf * kTF, m0 = tm * kTM;
  const int nk = static_cast<int>(p.K / kTK);

  // Loads: wave (wf, wt) fills rows 64 wt + 16 j .. + 15 (j < 4) of its group's
  // half of a stage, one 1 KB load each; lane L fills row 64 wt + 16 j + L / 4,
  // slot L % 4, with the row's chunk (L % 4) ^ swz(row).  The weight rows and
  // proj_in's token rows are read through a descriptor at the tile's first row
  // (lane offsets below 256 rows, the K step in the scalar offset); proj_out's
  // token rows through one at O (lane offset the row in O, scalar offset the
  // head and feature of the K step), or, for WIDE, through 64-bit addresses.
  constexpr bool LANE_PTR = MODE == 1 && WIDE;
  const bool tok_lane_ptr = LANE_PTR && wf == 1;
  const bf16_t* dbase = wf == 0 ? W + f0 * p.K : (MODE == 0 ? X + m0 * p.K : X);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)dbase, (short)0, -1, 0x00020000);
  uint32_t voff[4];
  const bf16_t* src[4];
  int ldst[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 64 * wt + 16 * j + (lane >> 2);
    const int chunk = (lane & 3) ^ swz(256 * wf + r);
    int64_t e;  // element offset of the row's chunk from dbase
    if (wf == 0) {
      e = (min(f0 + r, p.Nf - 1) - f0) * p.K;
    } else {
      const int64_t m = min(m0 + r, p.M - 1);
      if (MODE == 0) {
        e = (m - m0) * p.K;
      } else {
        const int64_t b = m / p.N, n = m - b * p.N;
        e = (b * p.H * p.N + n) * p.d;
      }
    }
    e += 8 * chunk;
    voff[j] = static_cast<uint32_t>(e * 2);
    if (LANE_PTR) src[j] = dbase + e;
    ldst[j] = (256 * wf + 64 * wt + 16 * j) * kTK;
  }
  // element offset of K step t: weights and proj_in tokens are contiguous in K;
  // proj_out tokens jump from head to head every d features
  auto k_off = [&](int t) -> int64_t {
    const int64_t k0 = static_cast<int64_t>(t) * kTK;
    if (MODE == 0 || wf == 0) return k0;
    return (k0 >> p.lgd) * p.N * p.d + (k0 & (p.d - 1));
  };
  // the ring's stage is a template argument (the loops below are unrolled by
  // the ring's depth), so stage offsets are immediates
  auto load_stage = [&](auto S, int t) {
    bf16_t* base = lds + decltype(S)::value * kStage;
    const int64_t off = k_off(t);
    if (tok_lane_ptr) {
#pragma unroll
      for (int j = 0; j < 4; ++j) global_to_lds16(src[j] + off, base + ldst[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) buffer_to_lds16(rs, base + ldst[j], voff[j], static_cast<int>(off * 2));
    }
  };
  // rows 128 wf + 32 fi + l32 and 256 + 64 wt + 32 ti + l32 have the swizzle of l32
  const int sw = swz(l32);
  bf16x8 a[4][2], bx[2][2];
  auto read_operands = [&](auto S) {
    const bf16_t* base = lds + decltype(S)::value * kStage;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = (2 * kk + h) ^ sw;
#pragma unroll
      for (int fi = 0; fi < 4; ++fi) {
        const int row = 128 * wf + 32 * fi + l32;
        a[fi][kk] = *reinterpret_cast<const bf16x8*>(base + row * kTK + 8 * c);
      }
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const int row = 256 + 64 * wt + 32 * ti + l32;
        bx[ti][kk] = *reinterpret_cast<const bf16x8*>(base + row * kTK + 8 * c);
      }
    }
  };
  f32x16 acc[4][2];
#pragma unroll
  for (int fi = 0; fi < 4; ++fi)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fi][ti][r] = 0.f;
  auto compute = [&]() {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
          acc[fi][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fi][kk], bx[ti][kk], acc[fi][ti], 0, 0, 0);
  };

  // Step t is loaded in phase pair t - 3 (the prologue loads steps 0-2) and read
  // by group 0 in the second phase of pair t - 1, by group 1 in the first phase
  // of pair t.  Before the barrier that precedes group 0's read, every wave waits
  // until at most its loads of later steps are outstanding (4 per step).
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  static_assert(kStages == 4, "the loops are unrolled by the ring's depth");
  const int pre = min(nk, 3);
  load_stage(S0{}, 0);
  if (pre > 1) load_stage(S1{}, 1);
  if (pre > 2) load_stage(S2{}, 2);
  if (pre == 3) {
    HA_WAIT_VMCNT(8);
  } else if (pre == 2) {
    HA_WAIT_VMCNT(4);
  } else {
    HA_WAIT_VMCNT(0);
  }
  phase_barrier();
  // step s of a group; U = s mod 4 (the stage step s occupies)
  auto step0 = [&](auto U, int s) {
    constexpr int u = decltype(U)::value;
    compute();
    if (s + 2 < nk) {
      HA_WAIT_VMCNT(4);  // step s + 2 may stay in flight
    } else {
      HA_WAIT_VMCNT(0);
    }
    phase_barrier();
    if (s + 1 < nk) read_operands(std::integral_constant<int, (u + 1) % 4>{});
    if (s + 3 < nk) load_stage(std::integral_constant<int, (u + 3) % 4>{}, s + 3);
    phase_barrier();
  };
  auto step1 = [&](auto U, int s) {
    constexpr int u = decltype(U)::value;
    read_operands(U);
    if (s + 3 < nk) {
      load_stage(std::integral_constant<int, (u + 3) % 4>{}, s + 3);
      HA_WAIT_VMCNT(8);  // steps s + 2 and s + 3 may stay in flight
    } else {
      HA_WAIT_VMCNT(0);
    }
    phase_barrier();
    compute();
    phase_barrier();
  };
  if (wf == 0) {
    read_operands(S0{});
    for (int s = 0; s < nk; s += 4) {
      step0(S0{}, s);
      if (s + 1 < nk) step0(S1{}, s + 1);
      if (s + 2 < nk) step0(S2{}, s + 2);
      if (s + 3 < nk) step0(S3{}, s + 3);
    }
  } else {
    for (int s = 0; s < nk; s += 4) {
      step1(S0{}, s);
      if (s + 1 < nk) step1(S1{}, s + 1);
      if (s + 2 < nk) step1(S2{}, s + 2);
      if (s + 3 < nk) step1(S3{}, s + 3);
    }
  }

  // epilogue: lane holds features f .. f+3 of token m for each (fi, ti, g).  A
  // 32-aligned run of features lies inside one head of one tensor (C and d are
  // multiples of 32), so each fi needs one 32-bit division by C.
  const int64_t C = MODE == 0 ? p.K : p.Nf;
  bf16_t* dst_fi[4];
  int64_t col_fi[4];
#pragma unroll
  for (int fi = 0; fi < 4; ++fi) {
    const int64_t fb = f0 + 128 * wf + 32 * fi;
    if (MODE == 0) {
      const uint32_t t = static_cast<uint32_t>(fb) / static_cast<uint32_t>(C);
      const int64_t fc = fb - static_cast<int64_t>(t) * C;
      dst_fi[fi] = t == 0 ? out0 : t == 1 ? out1 : t == 2 ? out2 : out3;
      col_fi[fi] = (fc >> p.lgd) * p.N * p.d + (fc & (p.d - 1));  // head offset + feature in head
    } else {
      dst_fi[fi] = out0;
      col_fi[fi] = fb;
    }
  }
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    const int64_t m = m0 + 64 * wt + 32 * ti + l32;
    if (m >= p.M) continue;
    int64_t row;  // element offset of token m's row
    if (MODE == 0) {
      const int64_t b = m / p.N, n = m - b * p.N;
      row = (b * p.H * p.N + n) * p.d;
    } else {
      row = m * C;
    }
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) {
      if (f0 + 128 * wf + 32 * fi >= p.Nf) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float v0 = acc[fi][ti][4 * g + 0], v1 = acc[fi][ti][4 * g + 1];
        const float v2 = acc[fi][ti][4 * g + 2], v3 = acc[fi][ti][4 * g + 3];
        const int64_t off = row + col_fi[fi] + 8 * g + 4 * h;
        if (MODE == 0) {
          *reinterpret_cast<uint2*>(dst_fi[fi] + off) = make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
        } else {
          const uint2 rv = *reinterpret_cast<const uint2*>(resid + off);
          *reinterpret_cast<uint2*>(out0 + off) =
              make_uint2(pack_bf16(bf_lo(rv.x) + v0, bf_hi(rv.x) + v1), pack_bf16(bf_lo(rv.y) + v2, bf_hi(rv.y) + v3));
        }
      }
    }
  }
}

// Plain float32 projections: 64 x 64 output tile per block of 256 threads,
// 4 x 4 outputs per thread, K through LDS in steps of 16.
template <int MODE>
__global__ __launch_bounds__(256) void proj_f32(const float* __restrict__ X, const float* __restrict__ W,
                                                float* out0, float* __restrict__ out1,
                                                float* __restrict__ out2, float* __restrict__ out3,
                                                const float* resid, ProjShape p) {
  __shared__ float sX[64][17];
  __shared__ float sW[64][17];
  const int tid = threadIdx.x;
  const int64_t nt_f = (p.Nf + 63) / 64;
  const int64_t tm = blockIdx.x / nt_f, tf = blockIdx.x % nt_f;
  const int64_t m0 = tm * 64, f0 = tf * 64;
  const int tx = tid & 15, ty = tid >> 4;  // features 4 tx.., tokens 4 ty..
  float acc[4][4] = {};
  auto xaddr = [&](int64_t m, int64_t k) -> int64_t {
    if (MODE == 0) return m * p.K + k;
    const int64_t b = m / p.N, n = m - b * p.N;
    return ((b * p.H + k / p.d) * p.N + n) * p.d + k % p.d;
  };
  for (int64_t k0 = 0; k0 < p.K; k0 += 16) {
    for (int e = tid; e < 64 * 16; e += 256) {
      const int r = e / 16, c = e % 16;
      const int64_t m = m0 + r, f = f0 + r, k = k0 + c;
      sX[r][c] = (m < p.M && k < p.K) ? X[xaddr(m, k)] : 0.f;
      sW[r][c] = (f < p.Nf && k < p.K) ? W[f * p.K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 16; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(sX[4 * ty + i][c], sW[4 * tx + j][c], acc[i][j]);
    __syncthreads();
  }
  const int64_t C = MODE == 0 ? p.K : p.Nf;
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + 4 * ty + i;
    if (m >= p.M) continue;
    const int64_t b = m / p.N, n = m - b * p.N;
    for (int j = 0; j < 4; ++j) {
      const int64_t f = f0 + 4 * tx + j;
      if (f >= p.Nf) continue;
      if (MODE == 0) {
        const int64_t t = f / C, fc = f - t * C;
        float* dst = t == 0 ? out0 : t == 1 ? out1 : t == 2 ? out2 : out3;
        dst[((b * p.H + fc / p.d) * p.N + n) * p.d + fc % p.d] = acc[i][j];
      } else {
        out0[m * C + f] = resid[m * C + f] + acc[i][j];
      }
    }
  }
}

ProjShape shape(int64_t B, int64_t H, int64_t N, int d, bool in) {
  ProjShape p{};
  const int64_t C = H * d;
  p.M = B * N;
  p.Nf = in ? 4 * C : C;
  p.K = C;
  p.N = N;
  p.H = H;
  p.d = d;
  p.lgd = d == 128 ? 7 : 6;
  p.nt_f = (p.Nf + kTF - 1) / kTF;
  p.nt_m = (p.M + kTM - 1) / kTM;
  p.total = p.nt_f * p.nt_m;
  return p;
}

template <int MODE>
hipError_t launch_proj(bool bf16, const void* X, const void* W, void* o0, void* o1, void* o2, void* o3,
                       const void* resid, int64_t B, int64_t H, int64_t N, int d, hipStream_t s) {
  const ProjShape p = shape(B, H, N, d, MODE == 0);
  if (p.M == 0 || p.K == 0) return hipSuccess;
  if (bf16) {
    auto go = [&](auto kern) {
      kern<<<dim3(static_cast<unsigned>(p.total)), dim3(512), 0, s>>>(
          static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(W), static_cast<bf16_t*>(o0),
          static_cast<bf16_t*>(o1), static_cast<bf16_t*>(o2), static_cast<bf16_t*>(o3),
          static_cast<const bf16_t*>(resid), p);
    };
    // proj_out's buffer offsets into O are 32-bit byte offsets from its start
    if constexpr (MODE == 1) {
      if (p.M * p.K * 2 >= (int64_t{1} << 32)) {
        go(proj_bf16<MODE, true>);
        return hipGetLastError();
      }
    }
    go(proj_bf16<MODE, false>);
  } else {
    const int64_t blocks = ((p.M + 63) / 64) * ((p.Nf + 63) / 64);
    proj_f32<MODE><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
        static_cast<const float*>(X), static_cast<const float*>(W), static_cast<float*>(o0),
        static_cast<float*>(o1), static_cast<float*>(o2), static_cast<float*>(o3),
        static_cast<const float*>(resid), p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proj_in(bool bf16, const void* x, const void* W_in, void* Q, void* K, void* V, void* G,
                          int64_t B, int64_t H, int64_t N, int d, hipStream_t s) {
  return launch_proj<0>(bf16, x, W_in, Q, K, V, G, nullptr, B, H, N, d, s);
}

hipError_t launch_proj_out(bool bf16, const void* O, const void* W_out, const void* x, void* x_out,
                           int64_t B, int64_t H, int64_t N, int d, hipStream_t s) {
  return launch_proj<1>(bf16, O, W_out, x_out, nullptr, nullptr, nullptr, x, B, H, N, d, s);
}

}  // namespace ha
