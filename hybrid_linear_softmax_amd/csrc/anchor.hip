// Gated softmax anchor (SANA-Video 2.0 summary page, section 03; review page,
// section 1): o_i = sigmoid(g_i) * sum_j softmax_j(q_i . k_j / sqrt(d)) v_j over
// all N tokens of the (batch, head), without materialising the N x N logits:
// key blocks stream through LDS and an online maximum and sum per query row
// rescale the running output (the flash-attention recurrence).
//
// bf16 kernel: one block = 256 queries of one (b, h), 8 waves x 32 queries
// (two waves per SIMD), 64 keys per iteration.
//  * logits are computed transposed, S^T = K Q^T, with the 32x32x16 bf16 MFMA:
//    the A operand is a K row from LDS, the B operand the wave's Q rows, held in
//    registers.  A lane's accumulator then holds 16 keys of ONE query, so the
//    row maximum and sum are lane-local except for one exchange with lane ^ 32;
//  * the probabilities P^T stay in registers and feed the PV MFMA directly as
//    its B operand (O^T += V^T P^T).  The key order that the accumulator layout
//    gives each lane is matched by storing V^T in LDS with bits 2 and 3 of the
//    key index swapped inside every 16-key group;
//  * V is transposed on its way into LDS (4 keys x 8 features per thread, one
//    v_perm per output dword); lanes are assigned so that the transposed 8-byte
//    stores of a wave fall on distinct LDS banks;
//  * K and V are read with buffer loads whose record count is the head's size:
//    rows past N read as zero without any per-load bounds arithmetic;
//  * software pipeline: the logit MFMAs of key block j+1 are interleaved, in
//    one wave's instruction stream, with the softmax of block j, then the PV
//    MFMAs of block j run with the next K/V fragments read ahead (the first
//    phase at raised wave priority); K and V tiles are double-
//    buffered in LDS, K one block ahead of V, one barrier per key block, and
//    the global loads of the next tiles are issued at the top of the step;
//  * the running maximum is updated lazily and without a per-block maximum: a
//    block's probabilities are computed against the running maximum m, and only
//    when some lane's sum of them exceeds 2^8 (so that a probability might) is
//    the block's exact maximum taken, the output and sums rescaled and the
//    block's probabilities recomputed.  Every probability that reaches the PV
//    product is therefore below 256 (exact enough in fp32 and bf16); after the
//    first blocks the slow path is almost never taken;
//  * row sums are taken over the bf16-rounded probabilities with v_dot2 (two per
//    instruction), i.e. over exactly the weights the PV product uses.  Each key
//    block is summed on its own and joins the running sum through compensated
//    (Kahan) addition: a lane's sum covers N/2 keys, and at millions of keys a
//    plain fp32 sum rounds every near-one pair the same way (its ulp reaches
//    0.5 past 2^22), which biases the denominator by about one percent.
#include <type_traits>

#include "ha_device.h"
#include "ha_launch.h"

namespace ha {

namespace {

constexpr int kBr = 256;  // queries per block (8 waves x 32)
constexpr int kBc = 64;   // keys per iteration
static_assert(kBr == kSparseBlockQ && kBc == kSparseBlockK, "sparse pattern blocks are the tile sizes");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSumLimit = 256.0f;  // a lane's block sum that triggers the exact rescale

// LDS column of key k (0..63 inside a key block) in the V^T tile.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// Block order of the sparse anchor: the blocks in flight all belong to one
// (b, h), spread over the 8 XCDs (blocks are dispatched round-robin), and each
// XCD walks a contiguous run of that head's query blocks.  Neighbouring query
// blocks share their local key windows in the XCD's L2, and every XCD reads the
// head's global frames, which then stay in the shared last-level cache.  (The
// dense anchor keeps xcd_remap: every query block reads every key there.)
__device__ __forceinline__ int64_t head_runs_remap(int64_t i, int64_t qblocks) {
  const int64_t hh = i / qblocks, j = i % qblocks, per = qblocks / 8;
  return hh * qblocks + (j < per * 8 ? (j % 8) * per + j / 8 : j);
}

// SPARSE: the query block walks the key blocks listed for it in a CSR pattern
// (blk_off / blk_idx) instead of all key blocks.  Listed indices outside
// [0, ceil(N/64)) are read as empty blocks (buffer loads past the head read
// zeros and every key is masked); offsets are clamped to [0, n_idx].
template <int D, bool SPARSE>
__global__ __launch_bounds__(512, 1) void anchor_bf16(const bf16_t* __restrict__ Q,
                                                      const bf16_t* __restrict__ K,
                                                      const bf16_t* __restrict__ V,
                                                      const bf16_t* __restrict__ G,
                                                      bf16_t* __restrict__ O, int64_t N,
                                                      int64_t qblocks, int64_t total, float c,
                                                      const int32_t* __restrict__ blk_off,
                                                      const int32_t* __restrict__ blk_idx,
                                                      int64_t n_idx, float* __restrict__ lse) {
  constexpr int NT = 512;
  constexpr int KP = D + 8;              // LDS pitch of K rows (elements)
  constexpr int VP = kBc + 8;            // LDS pitch of V^T rows (elements)
  constexpr int FG = D / 8;              // 16-byte groups per row
  constexpr int KCH = kBc * FG / NT;     // K chunks per thread per block
  constexpr int VSUB = (kBc / 4) * FG;   // V sub-tiles (4 keys x 8 features) per block
  constexpr int KS = D / 16;             // k-steps of the logit MFMA
  constexpr int RB = D / 32;             // 32-feature row blocks of O^T
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][kBc * KP];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[2][D * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int64_t id = SPARSE ? head_runs_remap(blockIdx.x, qblocks) : xcd_remap(blockIdx.x, total);
  const int64_t bh = id / qblocks;
  const int64_t q0 = (id % qblocks) * kBr + 32 * wave;
  const int64_t base = bh * N * D;
  const int64_t qrow = q0 + l32;
  const uint32_t head_bytes = static_cast<uint32_t>(N * D * 2);
  const __amdgpu_buffer_rsrc_t rK =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + base), (short)0, (int)head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rV =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + base), (short)0, (int)head_bytes, 0x00020000);

  // key blocks of this query block: dense 0 .. nkb-1, or the CSR list
  const int64_t nkb = (N + kBc - 1) / kBc;
  int64_t list_beg = 0, nsteps = nkb;
  if (SPARSE) {
    const int64_t qb = id % qblocks;
    list_beg = min(max((int64_t)blk_off[qb], (int64_t)0), n_idx);
    const int64_t list_end = min(max((int64_t)blk_off[qb + 1], list_beg), n_idx);
    nsteps = list_end - list_beg;
  }
  // (sparse) list entries are fetched with vector buffer loads two steps before
  // their use, so the wait for them is covered by the K/V loads in between;
  // loads past the list read 0 and are discarded by the i < nsteps test
  const __amdgpu_buffer_rsrc_t rL = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(SPARSE ? blk_idx + list_beg : blk_off), (short)0,
      SPARSE ? (int)(nsteps * 4) : 0, 0x00020000);
  auto fetch_entry = [&](int64_t i) -> int32_t {
    return __builtin_amdgcn_raw_buffer_load_b32(rL, (int)(min(i, nsteps) * 4), 0, 0);
  };
  // first key of step i's block; an absent or out-of-range block maps to a
  // past-the-end offset, whose loads read zeros and whose keys are all masked
  auto key0_of = [&](int64_t i, int32_t entry) -> int64_t {
    if (!SPARSE) return i * kBc;
    const int32_t e = __builtin_amdgcn_readfirstlane(entry);
    return (i < nsteps && e >= 0 && e < nkb) ? (int64_t)e * kBc : nkb * kBc;
  };
  auto block_valid = [&](int64_t k0) -> int { return static_cast<int>(min((int64_t)kBc, max((int64_t)0, N - k0))); };

  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = as_bf16x8(qrow < N ? *reinterpret_cast<const uint4*>(Q + base + qrow * D + 16 * s + 8 * h)
                               : make_uint4(0, 0, 0, 0));

  // V sub-tile of this thread: keys 4 v_m .. 4 v_m + 3, features 8 v_fg .. + 7;
  // consecutive lanes take consecutive key groups (distinct banks on store).
  const bool v_loader = tid < VSUB;
  const int v_fg = tid / 16, v_m = tid % 16;
  uint4 kreg[KCH], vreg[4];

  f32x16 o[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[rb][r] = 0.f;
  float m = -INFINITY;  // running max of the raw logits of this lane's query
  float lsum = 0.f;     // running sum of this lane's probabilities (half the keys)
  float lcomp = 0.f;    // its Kahan compensation: the low-order part lost so far

  // Software pipeline over 64-key blocks j: each step issues the logit MFMAs of
  // block j+1 (independent work) while the softmax of block j runs on the VALU,
  // then the PV MFMAs of block j.  K runs one block ahead of V in separate
  // double buffers.  The loop is unrolled by two so the two logit tiles swap
  // roles without register copies, and only the last steps carry the mask.
  auto qk = [&](int b, f32x16 (&s)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sK[b][(32 * t + l32) * KP + 16 * st + 8 * h]);
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s[t], 0, 0, 0);
      }
    }
  };
  auto mask = [&](f32x16 (&s)[2], int lim) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * t + 8 * (r >> 2) + 4 * h + (r & 3) >= lim) s[t][r] = -INFINITY;
  };
  auto rowmax = [&](const f32x16 (&s)[2]) {
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    return fmaxf(mx, __shfl_xor(mx, 32));
  };
  // raise the running maximum to m_new, rescaling what was summed against the
  // old one (alpha = 1 when it does not move, also while both are -inf)
  auto rescale_to = [&](float m_new) {
    const float alpha = m_new == m ? 1.f : __builtin_amdgcn_exp2f((m - m_new) * c);
    m = m_new;
    lsum *= alpha;
    lcomp *= alpha;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[rb][r] *= alpha;
  };
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  // K and V use separate double buffers; K runs one block ahead of V:
  // step j reads K_{j+1} (buffer (j+1)&1) and V_j (buffer j&1) and stores
  // K_{j+2} into K buffer j&1 and V_{j+1} into V buffer (j+1)&1.
  auto load_k = [&](int64_t kk0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int cidx = tid + NT * i;
      kreg[i] = buffer_load16(rK, static_cast<uint32_t>((kk0 + cidx / FG) * (D * 2) + (cidx % FG) * 16));
    }
  };
  auto load_v = [&](int64_t vk0) {
    if (v_loader) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = buffer_load16(rV, static_cast<uint32_t>((vk0 + 4 * v_m + r) * (D * 2) + v_fg * 16));
    }
  };
  auto store_kv = [&](int kb, int vb) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int cidx = tid + NT * i;
      *reinterpret_cast<uint4*>(&sK[kb][(cidx / FG) * KP + 8 * (cidx % FG)]) = kreg[i];
    }
    if (v_loader) {
      const int pos = vt_pos(4 * v_m);
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
      const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
      const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        *reinterpret_cast<uint2*>(&sVt[vb][(8 * v_fg + 2 * p) * VP + pos]) =
            make_uint2(__builtin_amdgcn_perm(r1[p], r0[p], 0x05040100u), __builtin_amdgcn_perm(r3[p], r2[p], 0x05040100u));
        *reinterpret_cast<uint2*>(&sVt[vb][(8 * v_fg + 2 * p + 1) * VP + pos]) =
            make_uint2(__builtin_amdgcn_perm(r1[p], r0[p], 0x07060302u), __builtin_amdgcn_perm(r3[p], r2[p], 0x07060302u));
      }
    }
  };
  // prologue: K_0, V_0 -> buffers 0, K_1 -> K buffer 1; S_0
  int32_t e1 = 0, e2 = 0;  // (sparse) list entries of steps j+1 and j+2
  if (SPARSE) {
    const int32_t e0 = fetch_entry(0);
    e1 = fetch_entry(1);
    e2 = fetch_entry(2);
    const int64_t k0 = key0_of(0, e0);
    load_k(k0);
    load_v(k0);
  } else {
    load_k(0);
    load_v(0);
  }
  store_kv(0, 0);
  load_k(key0_of(1, e1));
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int cidx = tid + NT * i;
    *reinterpret_cast<uint4*>(&sK[1][(cidx / FG) * KP + 8 * (cidx % FG)]) = kreg[i];
  }
  __syncthreads();
  f32x16 sa[2], sb[2];
  qk(0, sa);
  {
    const int lim = SPARSE ? block_valid(key0_of(0, fetch_entry(0))) : static_cast<int>(min((int64_t)kBc, N));
    if (lim < kBc) mask(sa, lim);
  }
  m = rowmax(sa);
  __syncthreads();
  // step j: k1, k2 are the first keys of blocks j+1 and j+2; masked steps
  // apply the key limit lim1 of block j+1 (in sparse mode only when it is
  // below 64).  The step is written in the order it should issue: each logit
  // MFMA of block j+1 is followed by two probabilities of block j (exp2, bf16
  // pack, row-sum dot), the first three PV MFMAs of block j by the compensated
  // addition of block j's probability sum, K/V fragments read two MFMAs ahead.
  // Empty asm statements that consume each result pin it between its MFMAs:
  // left alone, the compiler sinks the VALU work to its first use and clusters
  // the MFMAs.  Between the two phases, the rescale test on the block sums.
  auto step = [&](int64_t j, int64_t k1, int64_t k2, int lim1, f32x16 (&scur)[2], f32x16 (&snext)[2],
                  auto masked) {
    const int kb = static_cast<int>((j + 1) & 1);
    const int vb = static_cast<int>(j & 1);
    load_k(k2);
    load_v(k1);
    // the VALU-heavy phase runs at raised wave priority, the PV MFMAs at the
    // normal one (measured 1-2 % faster at 480p, 720p/5s and 14B)
    __builtin_amdgcn_s_setprio(2);
    // (sparse) while every key seen so far was masked, m = -inf: probabilities
    // are taken against 0 (masked keys give 0) and the first valid key forces
    // the exact rescale below
    float mc = (SPARSE && m == -INFINITY) ? 0.f : m * c;
    auto kfrag = [&](int i) -> bf16x8 {
      const int t = i & 1, st = i >> 1;
      return *reinterpret_cast<const bf16x8*>(&sK[kb][(32 * t + l32) * KP + 16 * st + 8 * h]);
    };
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) snext[t][r] = 0.f;
    constexpr int NQK = 2 * KS;          // logit MFMAs per block
    constexpr int PER = 16 / NQK;        // probability pairs per logit MFMA
    static_assert(PER * NQK == 16, "16 probability pairs per lane and block");
    bf16x8 kf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) kf[i] = kfrag(i);
    uint32_t pk[16];
    float lblk = 0.f;  // this block's probabilities, before they join lsum
    auto prob_pair = [&](int pi) {
      const int e0 = 2 * pi, e1 = e0 + 1;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(scur[e0 >> 4][e0 & 15], c, -mc));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(scur[e1 >> 4][e1 & 15], c, -mc));
      pk[pi] = pack_bf16(p0, p1);
      lblk = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[pi]), one, lblk, false);
    };
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int t = i & 1, st = i >> 1;
      const bf16x8 a = kf[i % 2];
      if (i + 2 < NQK) kf[i % 2] = kfrag(i + 2);
      snext[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], snext[t], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int pi = i * PER + u;
        prob_pair(pi);
        asm volatile("" : "+v"(pk[pi]), "+v"(lblk));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // a probability may exceed the limit only if the lane's block sum does (all
    // are non-negative); then take block j's exact maximum (its logits are
    // still in scur), rescale and recompute.  (sparse) the first block with a
    // valid key after masked ones always takes this path, so that m is finite
    // from then on.
    bool exact = lblk > kSumLimit;
    if (SPARSE) exact = exact || (m == -INFINITY && lblk > 0.f);
    if (__any(exact)) {
      rescale_to(fmaxf(m, rowmax(scur)));
      mc = (SPARSE && m == -INFINITY) ? 0.f : m * c;
      lblk = 0.f;
#pragma unroll
      for (int pi = 0; pi < 16; ++pi) prob_pair(pi);
    }
    // P^T operands: pf[t][tt] holds keys 32 t + 16 tt + (the accumulator's 8)
    bf16x8 pf[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        pf[t][tt] = as_bf16x8(make_uint4(pk[8 * t + 4 * tt], pk[8 * t + 4 * tt + 1], pk[8 * t + 4 * tt + 2],
                                         pk[8 * t + 4 * tt + 3]));
    if (decltype(masked)::value) {
      if (!SPARSE || lim1 < kBc) mask(snext, lim1);
    }
    __builtin_amdgcn_s_setprio(0);
    auto vfrag = [&](int i) -> bf16x8 {
      const int rb = i % RB, q = i / RB, t = q >> 1, tt = q & 1;
      return *reinterpret_cast<const bf16x8*>(&sVt[vb][(32 * rb + l32) * VP + 32 * t + 16 * tt + 8 * h]);
    };
    constexpr int NPV = 4 * RB;          // PV MFMAs per block
    bf16x8 vf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) vf[i] = vfrag(i);
    float ky, kt;  // Kahan terms of the block sum, spread over the first PV MFMAs
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int rb = i % RB, q = i / RB, t = q >> 1, tt = q & 1;
      const bf16x8 a = vf[i % 2];
      if (i + 2 < NPV) vf[i % 2] = vfrag(i + 2);
      o[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[t][tt], o[rb], 0, 0, 0);
      if (i == 0) { ky = lblk - lcomp; asm volatile("" : "+v"(ky)); }
      if (i == 1) { kt = lsum + ky; asm volatile("" : "+v"(kt)); }
      if (i == 2) { lcomp = (kt - lsum) - ky; lsum = kt; asm volatile("" : "+v"(lcomp), "+v"(lsum)); }
      __builtin_amdgcn_sched_barrier(0);
    }
    store_kv(static_cast<int>(j & 1), static_cast<int>((j + 1) & 1));
    __syncthreads();
  };
  using NoMask = std::integral_constant<bool, false>;
  using Mask = std::integral_constant<bool, true>;
  int64_t j = 0;
  if (!SPARSE) {
    // blocks 0 .. nfull-1 hold 64 valid keys: only the last steps mask
    const int64_t nfull = N / kBc;
    for (; j + 2 < nfull; j += 2) {
      step(j, (j + 1) * kBc, (j + 2) * kBc, kBc, sa, sb, NoMask{});
      step(j + 1, (j + 2) * kBc, (j + 3) * kBc, kBc, sb, sa, NoMask{});
    }
    for (; j < nsteps; j += 2) {
      step(j, (j + 1) * kBc, (j + 2) * kBc, block_valid((j + 1) * kBc), sa, sb, Mask{});
      if (j + 1 < nsteps) step(j + 1, (j + 2) * kBc, (j + 3) * kBc, block_valid((j + 2) * kBc), sb, sa, Mask{});
    }
  } else {
    auto sparse_step = [&](int64_t jj, f32x16 (&scur)[2], f32x16 (&snext)[2]) {
      const int64_t k1 = key0_of(jj + 1, e1);
      const int64_t k2 = key0_of(jj + 2, e2);
      e1 = e2;
      e2 = fetch_entry(jj + 3);
      step(jj, k1, k2, block_valid(k1), scur, snext, Mask{});
    };
    for (; j < nsteps; j += 2) {
      sparse_step(j, sa, sb);
      if (j + 1 < nsteps) sparse_step(j + 1, sb, sa);
    }
  }

  const float lrow = lsum - lcomp;
  const float l = lrow + __shfl_xor(lrow, 32);
  // (sparse) a query block with no valid key has l = 0 and gets O = 0
  const float inv = (SPARSE && !(l > 0.f)) ? 0.f : __builtin_amdgcn_rcpf(l);
  // natural log of sum_j exp(q . k_j / sqrt(d)) for the backward pass:
  // l is summed relative to exp2(m c), so lse = (m c + log2 l) ln 2
  if (lse != nullptr && qrow < N && h == 0) lse[bh * N + qrow] = (m * c + __log2f(l)) * kLn2;
  if (qrow < N) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int f0 = 32 * rb + 8 * g4 + 4 * h;
        const int64_t off = base + qrow * D + f0;
        const uint2 gv = *reinterpret_cast<const uint2*>(G + off);
        uint2 ov;
        ov.x = pack_bf16(gate_fast(bf_lo(gv.x)) * (o[rb][4 * g4 + 0] * inv),
                         gate_fast(bf_hi(gv.x)) * (o[rb][4 * g4 + 1] * inv));
        ov.y = pack_bf16(gate_fast(bf_lo(gv.y)) * (o[rb][4 * g4 + 2] * inv),
                         gate_fast(bf_hi(gv.y)) * (o[rb][4 * g4 + 3] * inv));
        *reinterpret_cast<uint2*>(O + off) = ov;
      }
  }
}

// Plain float32 anchor: two lanes per query (each half of d), 64 queries per
// block, 32-key blocks in LDS, online softmax per key block.  SPARSE walks the
// 64-key blocks listed for the enclosing 256-query block, as two 32-key halves.
template <int D, bool SPARSE>
__global__ __launch_bounds__(128) void anchor_f32(const float* __restrict__ Q,
                                                  const float* __restrict__ K,
                                                  const float* __restrict__ V,
                                                  const float* __restrict__ G,
                                                  float* __restrict__ O, int64_t N,
                                                  int64_t qblocks, float scale,
                                                  const int32_t* __restrict__ blk_off,
                                                  const int32_t* __restrict__ blk_idx,
                                                  int64_t n_idx, float* __restrict__ lse) {
  constexpr int BQ = 64, BK = 32, HD = D / 2;
  __shared__ float sK[BK][D];
  __shared__ float sV[BK][D];
  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int64_t bh = blockIdx.x / qblocks;
  const int64_t qrow = (blockIdx.x % qblocks) * BQ + (tid >> 1);
  const int64_t base = bh * N * D;
  float q[HD], acc[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    q[e] = qrow < N ? Q[base + qrow * D + half * HD + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  float lc = 0.f;  // Kahan compensation of l (the sum runs over up to N keys)
  const int64_t nkb = (N + kBc - 1) / kBc;
  int64_t list_beg = 0, nsteps = (N + BK - 1) / BK;
  if (SPARSE) {
    const int64_t qb = (blockIdx.x % qblocks) * BQ / kBr;
    list_beg = min(max((int64_t)blk_off[qb], (int64_t)0), n_idx);
    const int64_t list_end = min(max((int64_t)blk_off[qb + 1], list_beg), n_idx);
    nsteps = (list_end - list_beg) * (kBc / BK);
  }
  for (int64_t i = 0; i < nsteps; ++i) {
    int64_t k0 = i * BK;
    if (SPARSE) {
      const int64_t b = blk_idx[list_beg + i / (kBc / BK)];
      if (b < 0 || b >= nkb) continue;  // the same for every thread of the block
      k0 = b * kBc + (i % (kBc / BK)) * BK;
    }
    __syncthreads();
    for (int e = tid; e < BK * D; e += 128) {
      const int64_t key = k0 + e / D;
      sK[e / D][e % D] = key < N ? K[base + key * D + e % D] : 0.f;
      sV[e / D][e % D] = key < N ? V[base + key * D + e % D] : 0.f;
    }
    __syncthreads();
    float sc[BK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) part = fmaf(q[e], sK[j][half * HD + e], part);
      part += __shfl_xor(part, 1);
      sc[j] = k0 + j < N ? part * scale : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue;  // no valid key yet (sparse tail halves)
    const float alpha = expf(m - m_new);
    l *= alpha;
    lc *= alpha;
#pragma unroll
    for (int e = 0; e < HD; ++e) acc[e] *= alpha;
    float lb = 0.f;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      const float p = expf(sc[j] - m_new);
      lb += p;
#pragma unroll
      for (int e = 0; e < HD; ++e) acc[e] = fmaf(p, sV[j][half * HD + e], acc[e]);
    }
    const float y = lb - lc, t = l + y;
    lc = (t - l) - y;
    l = t;
    m = m_new;
  }
  l -= lc;
  if (lse != nullptr && qrow < N && half == 0) lse[bh * N + qrow] = m + logf(l);
  if (qrow < N) {
#pragma unroll
    for (int e = 0; e < HD; ++e) {
      const int64_t off = base + qrow * D + half * HD + e;
      O[off] = l > 0.f ? gate_exact(G[off]) * (acc[e] / l) : 0.f;
    }
  }
}

}  // namespace

hipError_t launch_anchor(bool bf16, int d, const void* Q, const void* K, const void* V,
                         const void* G, void* O, int64_t BH, int64_t N, hipStream_t s,
                         const int32_t* blk_off, const int32_t* blk_idx, int64_t n_idx, float* lse) {
  if (BH == 0 || N == 0) return hipSuccess;
  const bool sparse = blk_off != nullptr;
  if (bf16) {
    const int64_t qb = (N + kBr - 1) / kBr;
    const int64_t total = BH * qb;
    const float c = kLog2e / sqrtf(static_cast<float>(d));
    const bf16_t* q = static_cast<const bf16_t*>(Q);
    const bf16_t* k = static_cast<const bf16_t*>(K);
    const bf16_t* v = static_cast<const bf16_t*>(V);
    const bf16_t* g = static_cast<const bf16_t*>(G);
    bf16_t* o = static_cast<bf16_t*>(O);
    const dim3 grid(static_cast<unsigned>(total)), block(512);
    auto go = [&](auto kern) { kern<<<grid, block, 0, s>>>(q, k, v, g, o, N, qb, total, c, blk_off, blk_idx, n_idx, lse); };
    if (d == 128)
      sparse ? go(anchor_bf16<128, true>) : go(anchor_bf16<128, false>);
    else
      sparse ? go(anchor_bf16<64, true>) : go(anchor_bf16<64, false>);
  } else {
    const int64_t qb = (N + 63) / 64;
    const float scale = 1.0f / sqrtf(static_cast<float>(d));
    const float* q = static_cast<const float*>(Q);
    const float* k = static_cast<const float*>(K);
    const float* v = static_cast<const float*>(V);
    const float* g = static_cast<const float*>(G);
    float* o = static_cast<float*>(O);
    const dim3 grid(static_cast<unsigned>(BH * qb)), block(128);
    auto go = [&](auto kern) { kern<<<grid, block, 0, s>>>(q, k, v, g, o, N, qb, scale, blk_off, blk_idx, n_idx, lse); };
    if (d == 128)
      sparse ? go(anchor_f32<128, true>) : go(anchor_f32<128, false>);
    else
      sparse ? go(anchor_f32<64, true>) : go(anchor_f32<64, false>);
  }
  return hipGetLastError();
}

}  // namespace ha
