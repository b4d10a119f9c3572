// Grouped expert GEMMs on MFMA (gfx950).
//
// The experts are ungated ReLU^2 FFNs: an up part 2688 -> 1856 and a down
// part 1856 -> 2688 (bloomery issue #967, section 2 "Checkpoint facts" and
// section 3 "Existing owners and gaps"); rows routed to one expert are
// multiplied together (grouped expert matmul, audio.cpp notes, section "CPU
// weight offload").
//
// A workgroup computes a BM x BN tile of one expert: BM sorted rows of that
// expert (row tiles counted by the permutation on the device) times BN output
// columns.  Both operands are K-contiguous.  Four kernels:
//   grouped_gemm_kernel (BF16 and FP8 up-projection decode batches, 32-row
//     tiles): weight streaming; each thread loads 16-byte chunks two K steps
//     ahead into registers and stores them into double-buffered LDS (rows
//     padded to 144 bytes); FP8 up-projection codes are expanded on the way
//     into LDS.
//   grouped_gemm_rk_kernel (BF16 decode of a single expert whose grid is too
//     small to fill the chip: the shared expert): K split over the waves of
//     a workgroup, operands straight into registers, partial sums added
//     through LDS.
//   grouped_gemm_dma_kernel (BF16 and FP8 prefill, 128-row tiles, and the
//     FP8 down projection at decode, 32-row tiles): operands go from global
//     memory straight into LDS (global_load_lds_dwordx4) as stored, into an
//     XOR-swizzled layout; weight codes are expanded per lane when the MFMA
//     fragments are formed.  See the comment above that kernel.
//   grouped_gemm_nv_kernel (NVFP4, decode and prefill): packed weight codes
//     and block scales go from the panel layout straight into registers,
//     activations through LDS.
// Formats:
//   BF16 : v_mfma_f32_32x32x16_bf16, 64 K per step.
//   FP8  : v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales (E4M3 x
//          E4M3), 128 K per step; a 64-byte K tail (K = 1856 = 14*128 + 64)
//          is zeroed on chip rather than padded in HBM (zero padding of K
//          with matching zero activations leaves results unchanged: audio.cpp
//          notes, section "Q4_K, Q3_K and Q2_K expert profiles").
//   FP8X : E4M3 weight codes expanded to bf16 (v_cvt_scalef32_pk_bf16_fp8 with
//          unit scale, exact), then the BF16 MFMA on bf16 activations holding
//          dec(code).  Used for the FP8 up projection: the FP8 MFMA sums its 64
//          products with a short internal significand (about 13 bits below
//          the largest product), and the up projection's output is
//          re-quantised, so that error would move intermediate E4M3 codes;
//          exact products with fp32 sums do not.
//   NVFP4: E2M1 codes expanded to fp16 with v_cvt_scalef32_pk_f16_fp4 (unit
//          scale) and multiplied by the E4M3 block scale with v_pk_mul_f16:
//          code * block scale has at most 6 significant bits and lies in
//          [2^-10, 2688], so every fp16 value is exact; activations arrive as
//          the same exact fp16 products.  Then v_mfma_f32_32x32x16_f16 (exact
//          products, fp32 sums); the two fp32 tensor scales are applied in the
//          epilogue.  Codes and block scales are read in the bank's panel
//          layout (128-row panels, K-step-major), one contiguous block per
//          K step of a tile.
// Epilogues: up writes bf16(relu(h)^2) (and the tensor amax for quantised
// formats); down writes fp32 gate * h per sorted row.
#include <hip/hip_ext.h>
#include <type_traits>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kStepBytes = 128;  // K bytes of each A/B row staged per step
constexpr int kPrefetch = 2;     // K steps of loads in flight per thread
constexpr int kLds = 144;        // padded LDS row stride in bytes

// The expert that owns logical tile `logical`: the largest e in [0, E) with
// tile_off[e] * n_ntiles <= logical (tile_off is nondecreasing from
// tile_off[0] = 0, so that set of e is a prefix and its size less one is the
// answer).  Each lane tests up to four entries (E <= 256), all loaded in one
// round, and ballots count the entries at or below: one memory round trip
// before the tile's first loads instead of a dependent binary search.
__device__ __forceinline__ int owner_expert(const int32_t* __restrict__ tile_off, int E,
                                            int n_ntiles, int logical) {
  const int lane = threadIdx.x & 63;
  int v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ee = 1 + lane + 64 * q;
    v[q] = ee < E ? tile_off[ee] : 0;
  }
  int cnt = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ee = 1 + lane + 64 * q;
    cnt += __popcll(__ballot(ee < E && v[q] * n_ntiles <= logical));
  }
  return __builtin_amdgcn_readfirstlane(cnt);
}


template <int FMT, int STAGE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_kernel(GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int MB = WTM / 32, NB = WTN / 32;  // 32x32 MFMA blocks per wave
  // the FP8 down projection (fp8 MFMA) runs in grouped_gemm_dma_kernel and
  // NVFP4 in grouped_gemm_nv_kernel at every size
  static_assert(FMT == kBF16 || FMT == kFP8X, "BF16 and expanded FP8 only");
  // 16-byte source chunks per step: A rows 8 each, bf16 B rows 8 each (FP8
  // codes are loaded per pair of steps, below).  When a tile has fewer chunks
  // than threads, the extra threads repeat a chunk (same data to the same LDS
  // bytes), which keeps the loads branch-free.
  constexpr int A_TOT = BM * 8;
  constexpr int B_TOT = BN * 8;
  constexpr int A_CH = (A_TOT + NT - 1) / NT;
  constexpr int B_CH = (B_TOT + NT - 1) / NT;
  constexpr int ESZ = 2;  // bytes per staged element
  static_assert(MB >= 1 && NB >= 1 && A_CH >= 1 && B_CH >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (BM + BN) * kLds];
  uint8_t* const As = lds;
  uint8_t* const Bs = lds + 2 * BM * kLds;

  // ---- which tile.  Logical tiles run expert-major, then column tile, then
  // row tile, so one expert's activation rows and each weight panel are used
  // by tiles that run at the same time.  Blocks are dealt round-robin to the
  // 8 XCDs; each XCD takes a contiguous 1/8 of the logical tiles, so an
  // expert's rows and weights stay in one XCD's L2.
  const int n_ntiles = (g.N + BN - 1) / BN;
  const int total = g.tile_off[g.E] * n_ntiles;
  const int per_xcd = (total + 7) >> 3;
  const int local = blockIdx.x >> 3;
  if (local >= per_xcd) return;
  const int logical = (blockIdx.x & 7) * per_xcd + local;
  if (logical >= total) return;
  const int e = owner_expert(g.tile_off, g.E, n_ntiles, logical);
  const int te = g.tile_off[e + 1] - g.tile_off[e];
  const int loc = logical - g.tile_off[e] * n_ntiles;
  const int ntile = loc / te;
  const int mt = loc - ntile * te;
  const int row0 = g.offsets[e] + mt * BM;
  const int rows_valid = min(BM, g.offsets[e + 1] - row0);
  const int n0 = ntile * BN;
  // where the expert's weights sit: its own index, or its device cache slot
  const int ew = g.w_slot ? g.w_slot[e] : e;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int K = g.K, N = g.N;
  const int k_bytes = K * ESZ;
  const int n_steps = (k_bytes + kStepBytes - 1) / kStepBytes;

  // ---- per-thread global sources (fixed over K)
  const uint8_t* a_src[A_CH];
  int a_dst[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = (tid + i * NT) % A_TOT;
    const int r = c >> 3, cc = c & 7;
    const int rr = min(r, rows_valid - 1);
    size_t src;
    if constexpr (STAGE == 0) {
      src = static_cast<size_t>(g.sorted_src[row0 + rr] / g.top_k);
    } else {
      src = static_cast<size_t>(row0 + rr);
    }
    a_src[i] = static_cast<const uint8_t*>(g.a) + src * k_bytes + cc * 16;
    a_dst[i] = r * kLds + cc * 16;
  }
  const uint8_t* b_src[B_CH];
  int b_dst[B_CH];
  if constexpr (FMT == kBF16) {
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = (tid + i * NT) % B_TOT;
      const int r = c >> 3, cc = c & 7;
      const int n = min(n0 + r, N - 1);
      const size_t row = static_cast<size_t>(ew) * N + n;
      b_src[i] = static_cast<const uint8_t*>(g.b) + row * k_bytes + cc * 16;
      b_dst[i] = r * kLds + cc * 16;
    }
  }
  // Expanded FP8 codes: one K step is 64 codes, half of a 128-byte line of a
  // weight row.  Their loads cover pairs of steps so that the 8 lanes of a row
  // read its whole line in one instruction: lane bit 2, flipped on odd
  // chunks, picks the half, so each thread holds two chunks of each step.
  constexpr int B_PCH = (FMT == kFP8X) ? BN * 8 / NT : 2;
  static_assert(FMT != kFP8X || (BN * 8 % NT == 0 && NT % 8 == 0 && B_PCH % 2 == 0),
                "fp8 pair chunks");
  const int h0 = (tid >> 2) & 1;
  const uint8_t* bp_row[B_PCH];
  int bp_dst[B_PCH];
  if constexpr (FMT == kFP8X) {
#pragma unroll
    for (int i = 0; i < B_PCH; ++i) {
      const int c = tid + i * NT;
      const int r = c >> 3, q = c & 3;
      const int n = min(n0 + r, N - 1);
      const size_t row = static_cast<size_t>(ew) * N + n;
      bp_row[i] = static_cast<const uint8_t*>(g.b) + row * K + q * 16;
      bp_dst[i] = r * kLds + q * 32;
    }
  }

  // two register sets: the loads of steps s+1 and s+2 are in flight while
  // step s is multiplied out of LDS (FP8 codes: two sets of step pairs)
  u32x4 a_reg[kPrefetch][A_CH];
  u32x4 b_reg[kPrefetch][B_CH];
  u32x4 bp_reg[2][B_PCH];

  // BF16: steps past the end are not loaded (a wave-uniform branch).
  // Re-reading the last step there cost 2-7 % of a decode launch: the
  // non-temporal weight lines are not kept for a second read.  Expanded FP8
  // codes: steps past the end re-read the last step (no branches around the
  // loads; a branch there made the compiler wait for more than the set it
  // needs, 5-25 % slower).  K is a multiple of 64, so bf16 rows hold whole
  // 128-byte steps.
  auto load = [&](int step_in, auto set_c, auto nt_c) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_c)::value;
    constexpr bool NT = decltype(nt_c)::value;
    if constexpr (FMT == kBF16) {
      if (step_in >= n_steps) return;
    }
    const int step = min(step_in, n_steps - 1);
    const int kb = step * kStepBytes;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) a_reg[SET][i] = *reinterpret_cast<const u32x4*>(a_src[i] + kb);
    if constexpr (FMT == kBF16) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        if constexpr (NT) {
          b_reg[SET][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b_src[i] + kb));
        } else {
          b_reg[SET][i] = *reinterpret_cast<const u32x4*>(b_src[i] + kb);
        }
      }
    }
  };

  // FP8 codes of K steps 2 pair and 2 pair + 1 into pair set PS (a step past
  // the end re-reads the last one)
  auto load_pair = [&](int pair, auto ps_c, auto nt_c) __attribute__((always_inline)) {
    constexpr int PS = decltype(ps_c)::value;
    constexpr bool NT = decltype(nt_c)::value;
#pragma unroll
    for (int i = 0; i < B_PCH; ++i) {
      const int step = min(2 * pair + (h0 ^ (i & 1)), n_steps - 1);
      const u32x4* p = reinterpret_cast<const u32x4*>(bp_row[i] + step * 64);
      if constexpr (NT) {
        bp_reg[PS][i] = __builtin_nontemporal_load(p);
      } else {
        bp_reg[PS][i] = *p;
      }
    }
  };

  // 16 E4M3 codes -> 16 bf16 (unit scale: exact), 32 bytes at dst
  auto expand_fp8 = [&](uint8_t* dst_b, const u32x4 v) __attribute__((always_inline)) {
    uint32_t outw[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[w], 1.0f, false);
      const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[w], 1.0f, true);
      outw[2 * w] = __builtin_bit_cast(uint32_t, lo);
      outw[2 * w + 1] = __builtin_bit_cast(uint32_t, hi);
    }
    // Lanes 4-7 of each group of eight write a row 32 rows below lanes 0-3,
    // which sits on the same LDS banks (32 rows of 144 bytes are a multiple
    // of the bank period).  They write their 32 bytes in the other order, so
    // each store instruction's eight lanes cover distinct banks (bank
    // conflicts 88 % of LDS cycles -> 0).
    u32x4* dst = reinterpret_cast<u32x4*>(dst_b);
    const u32x4 first = u32x4{outw[0], outw[1], outw[2], outw[3]};
    const u32x4 second = u32x4{outw[4], outw[5], outw[6], outw[7]};
    dst[h0] = h0 ? second : first;
    dst[h0 ^ 1] = h0 ? first : second;
  };

  // the half HS (0: even step, 1: odd step) of pair set PS into buffer buf
  auto store_pair = [&](int buf, auto ps_c, auto hs_c) __attribute__((always_inline)) {
    constexpr int PS = decltype(ps_c)::value;
    constexpr int HS = decltype(hs_c)::value;
    uint8_t* B = Bs + buf * BN * kLds;
    const bool odd = (h0 ^ HS) != 0;  // this thread's chunks 2j + 1 hold that step
#pragma unroll
    for (int j = 0; j < B_PCH / 2; ++j) {
      // select values, not array elements, so the arrays stay in registers
      const u32x4 e = bp_reg[PS][2 * j], o = bp_reg[PS][2 * j + 1];
      const int de = bp_dst[2 * j], dodd = bp_dst[2 * j + 1];
      u32x4 v;
#pragma unroll
      for (int w = 0; w < 4; ++w) v[w] = odd ? o[w] : e[w];
      expand_fp8(B + (odd ? dodd : de), v);
    }
  };

  auto store = [&](int buf, auto set_c) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_c)::value;
    uint8_t* A = As + buf * BM * kLds;
    uint8_t* B = Bs + buf * BN * kLds;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) *reinterpret_cast<u32x4*>(A + a_dst[i]) = a_reg[SET][i];
    if constexpr (FMT == kBF16) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) *reinterpret_cast<u32x4*>(B + b_dst[i]) = b_reg[SET][i];
    }
  };

  // ---- which MFMA blocks of this wave hold live rows / columns.  Row blocks
  // past the expert's last row are skipped: the main loop is specialised on
  // the number of live 32-row blocks of the wave (a wave-uniform value), so the
  // padding of ragged experts costs no MFMA issue and no branches in the loop.
  // Dead columns (past N) hold clamped copies of live ones and are only masked
  // in the epilogue.
  // Row blocks are dealt to the WM wave rows in turn (wave row wm owns 32-row
  // blocks wm, wm + WM, ...), so a ragged tile's live blocks spread evenly
  // over the waves, and waves sharing a SIMD get equal work.
  const int live_blocks = (rows_valid + 31) >> 5;
  int ml_raw = (live_blocks - wm + WM - 1) / WM;
  ml_raw = ml_raw < 0 ? 0 : (ml_raw > MB ? MB : ml_raw);
  const int ml = __builtin_amdgcn_readfirstlane(ml_raw);
  bool n_live[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) n_live[j] = n0 + wn * WTN + j * 32 < N;

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31;
  const int lk = lane >> 5;  // which K half of a sub-step this lane supplies

  // multiply the first ML row blocks of the wave out of LDS buffer buf
  auto compute = [&](int buf, auto ml_c) __attribute__((always_inline)) {
    constexpr int ML = decltype(ml_c)::value;
    if constexpr (ML > 0) {
      const uint8_t* A = As + buf * BM * kLds;
      const uint8_t* B = Bs + buf * BN * kLds;
      using frag = bf16x8;
      // fragments of sub-step s+1 are read while the MFMAs of sub-step s run
      frag af[2][ML], bfr[2][NB];
      auto rd = [&](int s, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < ML; ++i)
          af[slot][i] = *reinterpret_cast<const frag*>(
              A + ((i * WM + wm) * 32 + lrow) * kLds + s * 32 + lk * 16);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          bfr[slot][j] = *reinterpret_cast<const frag*>(
              B + (wn * WTN + j * 32 + lrow) * kLds + s * 32 + lk * 16);
      };
      rd(0, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {  // 16 K per MFMA
        if (s < 3) rd(s + 1, (s + 1) & 1);
#pragma unroll
        for (int i = 0; i < ML; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][i], bfr[s & 1][j],
                                                                acc[i][j], 0, 0, 0);
      }
    }
  };

  // ---- main loop: one barrier per K step, double-buffered LDS, loads two
  // steps ahead in two register sets.  Unrolled by two so register sets are
  // compile-time indices; a trailing iteration past the last step stores
  // into a buffer that is not read again and computes nothing.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto main_loop = [&](auto ml_c, auto nt_c) __attribute__((always_inline)) {
    auto iter = [&](int step, auto set_next) __attribute__((always_inline)) {
      // data of step+1 sits in register set (step+1) % 2 == set_next
      if (step < n_steps) compute(step & 1, ml_c);
      store((step + 1) & 1, set_next);
      load(step + 1 + kPrefetch, set_next, nt_c);
      __syncthreads();
    };
    load(0, S0{}, nt_c);
    load(1, S1{}, nt_c);
    store(0, S0{});
    load(2, S0{}, nt_c);
    __syncthreads();
    for (int step = 0; step < n_steps; step += 2) {
      iter(step, S1{});
      iter(step + 1, S0{});
    }
  };
  // FP8 codes: activations per step as above; codes per pair of steps, two
  // pair sets, so the loads of a pair are issued three steps before its first
  // step is stored.  Unrolled by four (A set, pair set and half are
  // compile-time); the loop stops after the iteration that computes the last
  // step.
  using F0 = std::false_type;
  using T1 = std::true_type;
  auto main_loop_pairs = [&](auto ml_c, auto nt_c) __attribute__((always_inline)) {
    // iteration `step` computes step, then stages step + 1: its activations
    // from set a_next, its codes from pair set ps, half hs
    auto iter = [&](int step, auto a_next, auto ps, auto hs, auto reload) __attribute__((always_inline)) {
      if (step < n_steps) compute(step & 1, ml_c);
      store((step + 1) & 1, a_next);
      store_pair((step + 1) & 1, ps, hs);
      load(step + 1 + kPrefetch, a_next, nt_c);
      // both halves of pair set ps are staged: refill it two pairs ahead
      if constexpr (decltype(reload)::value) load_pair((step + 1) / 2 + 2, ps, nt_c);
      __syncthreads();
    };
    load(0, S0{}, nt_c);
    load(1, S1{}, nt_c);
    load_pair(0, S0{}, nt_c);
    load_pair(1, S1{}, nt_c);
    store(0, S0{});
    store_pair(0, S0{}, S0{});
    load(2, S0{}, nt_c);
    __syncthreads();
    for (int step = 0; step < n_steps; step += 4) {
      iter(step, S1{}, S0{}, S1{}, T1{});
      if (step + 1 >= n_steps) break;
      iter(step + 1, S0{}, S1{}, S0{}, F0{});
      if (step + 2 >= n_steps) break;
      iter(step + 2, S1{}, S1{}, S1{}, T1{});
      if (step + 3 >= n_steps) break;
      iter(step + 3, S0{}, S0{}, S0{}, F0{});
    }
  };
  static_assert(MB <= 8, "row blocks per wave");
  auto run = [&](auto nt_c) __attribute__((always_inline)) {
    auto go = [&](auto ml_c) __attribute__((always_inline)) {
      if constexpr (FMT == kFP8X) main_loop_pairs(ml_c, nt_c);
      else main_loop(ml_c, nt_c);
    };
    switch (ml) {
      case 0: go(std::integral_constant<int, 0>{}); break;
      case 1: go(std::integral_constant<int, (MB >= 1 ? 1 : MB)>{}); break;
      case 2: go(std::integral_constant<int, (MB >= 2 ? 2 : MB)>{}); break;
      case 3: go(std::integral_constant<int, (MB >= 3 ? 3 : MB)>{}); break;
      case 4: go(std::integral_constant<int, (MB >= 4 ? 4 : MB)>{}); break;
      case 5: go(std::integral_constant<int, (MB >= 5 ? 5 : MB)>{}); break;
      case 6: go(std::integral_constant<int, (MB >= 6 ? 6 : MB)>{}); break;
      case 7: go(std::integral_constant<int, (MB >= 7 ? 7 : MB)>{}); break;
      default: go(std::integral_constant<int, MB>{}); break;
    }
  };
  // Weight panels that only this workgroup reads (the expert has one row
  // tile) stream through with non-temporal loads: BF16 7-8 % faster at 4 to
  // 128 tokens.  Panels that sibling row tiles re-read keep ordinary loads,
  // which leave the lines in L2 for them (non-temporal loads there were
  // 5-10 % slower at 384 and 511 tokens).
  if (te == 1) run(T1{});
  else run(F0{});

  // ---- epilogue.  32x32 f32 result: lane holds column lane%32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
  // scales of the quantised formats: s_act * s_weight (exact in double),
  // rounded once to fp32
  double scale = 1.0;
  if constexpr (FMT != kBF16) scale = static_cast<double>(g.a_s[0]) * static_cast<double>(g.b_s[e]);
  const float scale_f = static_cast<float>(scale);
  float local_max = 0.f;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if (i >= ml) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (!n_live[j]) continue;
      const int col = n0 + wn * WTN + j * 32 + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = (i * WM + wm) * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
        if (rl < rows_valid && col < N) {
          const size_t at = static_cast<size_t>(row0 + rl) * N + col;
          if constexpr (STAGE == 0) {
            // a = bf16(relu(h)^2), rounded once from the exact square of the
            // fp32 h (BF16: the accumulator itself)
            float h = acc[i][j][r];
            if constexpr (FMT != kBF16) h *= scale_f;
            const uint16_t b = relu_sq_bf16(h);
            static_cast<uint16_t*>(g.out)[at] = b;
            if constexpr (FMT != kBF16) local_max = fmaxf(local_max, bf16_to_f32(b));
          } else {
            const float gate = g.row_gate[row0 + rl];
            float o;
            if constexpr (FMT == kBF16) {
              o = acc[i][j][r] * gate;
            } else {
              o = acc[i][j][r] * (scale_f * gate);
            }
            static_cast<float*>(g.out)[at] = o;
          }
        }
      }
    }
  }
  if constexpr (STAGE == 0 && FMT != kBF16) block_amax_to_slots(local_max, g.amax);
}

// ---------------------------------------------------------------------------
// BF16 decode kernel for grids too small to fill the chip (one expert, a few
// row tiles: the shared expert at decode).  The kernels above give each
// workgroup a whole K loop, so a grid of a few dozen workgroups keeps a few
// dozen waves' loads in flight.  Here a workgroup of KS waves computes one
// 32 x 32 tile and wave w takes the K steps w, w + KS, w + 2 KS, ...: KS
// times more waves stream the same weights.  Both operands go straight into
// registers (a ring of P steps of loads in flight per wave; no LDS and no
// barrier in the K loop), and the waves' fp32 partial sums are added through
// LDS in wave order at the end, so results do not depend on timing.
//
// A step is 64 K: sub-step q multiplies K 16 q .. 16 q + 15, the lane half
// lk supplying its 8 values at 16 q + 8 lk (the MFMA's own K order), so one
// load instruction reads 32 contiguous bytes of each of 32 rows.  Ordinary
// loads: with the non-temporal policy each line was dropped before the next
// instruction read its other bytes, at half the speed.
template <int STAGE, int KS, int P>
__global__ __launch_bounds__(KS * 64) void grouped_gemm_rk_kernel(GemmArgs g) {
  static_assert(KS >= 1 && KS <= 8 && P >= 1 && P <= 4, "split and depth");
  constexpr int BM = 32, BN = 32;
  __shared__ f32x4 part[KS > 1 ? (KS - 1) * 4 * 64 : 1];

  // ---- which tile (same order as the kernels above)
  const int n_ntiles = (g.N + BN - 1) / BN;
  const int total = g.tile_off[g.E] * n_ntiles;
  const int per_xcd = (total + 7) >> 3;
  const int local = blockIdx.x >> 3;
  if (local >= per_xcd) return;
  const int logical = (blockIdx.x & 7) * per_xcd + local;
  if (logical >= total) return;
  const int e = owner_expert(g.tile_off, g.E, n_ntiles, logical);
  const int te = g.tile_off[e + 1] - g.tile_off[e];
  const int loc = logical - g.tile_off[e] * n_ntiles;
  const int ntile = loc / te;
  const int mt = loc - ntile * te;
  const int row0 = g.offsets[e] + mt * BM;
  const int rows_valid = min(BM, g.offsets[e + 1] - row0);
  const int n0 = ntile * BN;
  const int ew = g.w_slot ? g.w_slot[e] : e;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 31, lk = lane >> 5;
  const int K = g.K, N = g.N;
  const size_t row_bytes = static_cast<size_t>(K) * 2;
  const int n_steps = K / 64;  // K is a multiple of 64
  // this wave's steps; a wave with none (K shorter than KS steps) adds zeros
  const int n_my = n_steps > wave ? (n_steps - wave + KS - 1) / KS : 0;

  // rows past the tile's last one read that row again, columns past N the
  // last column; both are masked in the epilogue
  const int rr = min(lrow, rows_valid - 1);
  size_t src;
  if constexpr (STAGE == 0) {
    src = static_cast<size_t>(g.sorted_src[row0 + rr] / g.top_k);
  } else {
    src = static_cast<size_t>(row0 + rr);
  }
  const int n = min(n0 + lrow, N - 1);
  const uint8_t* a_ptr = static_cast<const uint8_t*>(g.a) + src * row_bytes + wave * 128 + lk * 16;
  const uint8_t* b_ptr = static_cast<const uint8_t*>(g.b) +
                         (static_cast<size_t>(ew) * N + n) * row_bytes + wave * 128 + lk * 16;
  constexpr int kStride = KS * 128;  // bytes between a wave's consecutive steps

  u32x4 ra[P][4], rb[P][4];
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  // the wave's step j into ring slot SLOT
  auto load = [&](int j, auto slot_c) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_c)::value;
    const size_t off = static_cast<size_t>(j) * kStride;
    const u32x4* pa = reinterpret_cast<const u32x4*>(a_ptr + off);
    const u32x4* pb = reinterpret_cast<const u32x4*>(b_ptr + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[SLOT][q] = pa[2 * q];
      rb[SLOT][q] = pb[2 * q];
    }
  };
  auto compute = [&](auto slot_c) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_c)::value;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ra[SLOT][q]),
                                                    __builtin_bit_cast(bf16x8, rb[SLOT][q]), acc,
                                                    0, 0, 0);
  };
  // steps j0 .. j0 + P - 1 from the ring, each slot refilled P steps ahead
  // (no loads past the wave's last step)
  auto prime = [&](auto slot_c) __attribute__((always_inline)) {
    if (decltype(slot_c)::value < n_my) load(decltype(slot_c)::value, slot_c);
  };
  prime(std::integral_constant<int, 0>{});
  if constexpr (P >= 2) prime(std::integral_constant<int, 1>{});
  if constexpr (P >= 3) prime(std::integral_constant<int, 2>{});
  if constexpr (P >= 4) prime(std::integral_constant<int, 3>{});
  for (int j0 = 0; j0 < n_my; j0 += P) {
    auto one = [&](auto slot_c) __attribute__((always_inline)) {
      constexpr int SLOT = decltype(slot_c)::value;
      const int j = j0 + SLOT;
      if (j < n_my) compute(slot_c);
      if (j + P < n_my) load(j + P, slot_c);
    };
    one(std::integral_constant<int, 0>{});
    if constexpr (P >= 2) one(std::integral_constant<int, 1>{});
    if constexpr (P >= 3) one(std::integral_constant<int, 2>{});
    if constexpr (P >= 4) one(std::integral_constant<int, 3>{});
  }

  // ---- partial sums of waves 1 .. KS - 1 through LDS, added in wave order
  if constexpr (KS > 1) {
    if (wave > 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        part[((wave - 1) * 4 + q) * 64 + lane] =
            f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = part[(w * 4 + q) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * q + i] += v[i];
      }
  }

  // ---- epilogue (wave 0).  Lane holds column lane % 32 and rows
  // 8 (r / 4) + 4 (lane / 32) + r % 4.
  const int col = n0 + lrow;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rl = (r >> 2) * 8 + lk * 4 + (r & 3);
    if (rl < rows_valid && col < N) {
      const size_t at = static_cast<size_t>(row0 + rl) * N + col;
      if constexpr (STAGE == 0) {
        static_cast<uint16_t*>(g.out)[at] = relu_sq_bf16(acc[r]);
      } else {
        static_cast<float*>(g.out)[at] = acc[r] * g.row_gate[row0 + rl];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill kernel with direct global -> LDS loads (global_load_lds_dwordx4).
// Per-thread ds_write staging costs about as much LDS time as all the
// fragment reads of a K step on this part; direct loads move each 16-byte
// chunk from L1 into LDS without passing through VGPRs.  Operands are staged
// as stored: bf16 / E4M3 activations and bf16 weights or E4M3 weight codes;
// codes of the up projection are expanded per lane when the MFMA fragments
// are formed.
//
// LDS holds NBUF buffers of one K step: BM activation rows of 128 bytes and
// BN weight rows of RB bytes (128 bf16 / fp8, 64 fp8 codes expanded to
// bf16).  Rows are not
// padded: chunk c (16 bytes) of row r sits in slot c ^ ((r / (256 / RB)) %
// (RB / 16)), so the 16 rows that a quarter-wave ds_read_b128 touches at one
// chunk land on distinct banks.  A direct load writes one wave's 64 x 16
// bytes to consecutive LDS addresses; each lane fetches the global chunk that
// belongs in its slot.  Loads run NBUF - 1 steps ahead; at the top of each
// step a wave waits for its own loads of that step (vmcnt) and the workgroup
// meets at a barrier, after which every wave's loads are visible.
//
// K order inside a step: BF16 and FP8 feed the MFMA in natural order.  For
// expanded FP8 codes lane half lk takes the step's K range [32 lk, 32 lk +
// 32) and sub-step s its 8 values at 32 lk + 8 s, so one lane's codes are
// contiguous; activations are read in the same order (a permutation of K
// inside the step, which the exact products and fp32 sums do not notice
// beyond summation order).

template <int RB>
__device__ __forceinline__ int lds_swz(int r) {
  return (r / (256 / RB)) % (RB / 16);
}

// s_waitcnt immediate that waits until at most n vector memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

template <int FMT, int STAGE, int BM, int BN, int WM, int WN, int NBUF>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_dma_kernel(GemmArgs g) {
  static_assert(NBUF >= 2 && NBUF <= 4, "buffers");
  static_assert(FMT == kBF16 || FMT == kFP8 || FMT == kFP8X, "bf16, fp8 or expanded fp8");
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;
  constexpr bool EXPAND = FMT == kFP8X;
  constexpr int AESZ = (FMT == kFP8) ? 1 : 2;           // activation bytes per element
  constexpr int KS = 128 / AESZ;                         // K elements per step
  constexpr int RB = (FMT == kFP8X) ? 64 : 128;          // weight row bytes per step
  constexpr int NA = BM / 8;                             // activation loads per step (8 rows each)
  constexpr int NBL = BN * RB / 1024;                    // weight loads per step
  constexpr int QA = (NA + NW - 1) / NW, QB = (NBL + NW - 1) / NW;
  constexpr int DPS = QA + QB;                           // vector memory operations per wave per step
  constexpr int A_OFF = 0, B_OFF = BM * 128;
  constexpr int BUF = BM * 128 + BN * RB;
  static_assert(NA * 8 == BM && NBL * 1024 == BN * RB && BM % 16 == 0 && BN % 64 == 0, "tile");
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[NBUF >= 3 ? BUF : 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[NBUF >= 4 ? BUF : 1024];

  // ---- which tile (same order as grouped_gemm_kernel)
  const int n_ntiles = (g.N + BN - 1) / BN;
  const int total = g.tile_off[g.E] * n_ntiles;
  const int per_xcd = (total + 7) >> 3;
  const int local = blockIdx.x >> 3;
  if (local >= per_xcd) return;
  const int logical = (blockIdx.x & 7) * per_xcd + local;
  if (logical >= total) return;
  const int e = owner_expert(g.tile_off, g.E, n_ntiles, logical);
  const int te = g.tile_off[e + 1] - g.tile_off[e];
  const int loc = logical - g.tile_off[e] * n_ntiles;
  const int ntile = loc / te;
  const int mt = loc - ntile * te;
  const int row0 = g.offsets[e] + mt * BM;
  const int rows_valid = min(BM, g.offsets[e + 1] - row0);
  const int n0 = ntile * BN;
  // where the expert's weights sit: its own index, or its device cache slot
  const int ew = g.w_slot ? g.w_slot[e] : e;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int K = g.K, N = g.N;
  const int a_bytes = K * AESZ;                 // activation row bytes
  const int w_bytes = (FMT == kBF16) ? 2 * K : K;       // weight row bytes
  const int n_steps = (K + KS - 1) / KS;

  // ---- per-lane global sources of the direct loads (fixed over K).  When a
  // load class has fewer instructions than waves, waves repeat one (same
  // source, same LDS bytes) so every wave issues DPS loads per step.
  const uint8_t* a_src[QA];
  int a_dst[QA], a_cof[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int qi = (wave + q * NW) % NA;
    const int r = qi * 8 + (lane >> 3);
    const int c = (lane & 7) ^ lds_swz<128>(r);
    const int rr = min(r, rows_valid - 1);
    size_t src;
    if constexpr (STAGE == 0) {
      src = static_cast<size_t>(g.sorted_src[row0 + rr] / g.top_k);
    } else {
      src = static_cast<size_t>(row0 + rr);
    }
    a_src[q] = static_cast<const uint8_t*>(g.a) + src * a_bytes + c * 16;
    a_dst[q] = A_OFF + qi * 1024;
    a_cof[q] = c * 16;
  }
  constexpr int CPR = RB / 16;  // 16-byte chunks per weight row and step
  // FP8 down-projection codes sit in panels stored
  // K-step-major (the tile lies inside one panel): a step of the tile's rows
  // is contiguous, w_step bytes apart.  FP8 steps are whole 128-byte lines;
  // when K % 128 == 64 the last step holds 64 bytes per row, and its chunks
  // move by b_tail[q] (chunks past K re-read the row's in-range chunk 64
  // bytes earlier and are zeroed when the fragments are formed).
  constexpr bool kPanels = FMT == kFP8;
  static_assert(!kPanels || kNvPanel % BN == 0, "panel-layout tiles stay inside one panel");
  static_assert(FMT != kFP8 || RB == kFp8StepK, "fp8 panel steps");
  const int nv_pn0 = n0 - n0 % kNvPanel;
  const int nv_rows = nv_panel_rows(N, nv_pn0 / kNvPanel);
  const int w_step = kPanels ? nv_rows * RB : RB;
  const bool fp8_tail_step = FMT == kFP8 && (K % RB) != 0;
  const uint8_t* b_src[QB];
  int b_dst[QB], b_tail[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int qi = (wave + q * NW) % NBL;
    const int r = qi * (1024 / RB) + lane / CPR;
    const int c = (lane % CPR) ^ lds_swz<RB>(r);
    const int n = min(n0 + r, N - 1);
    if constexpr (kPanels) {
      b_src[q] = static_cast<const uint8_t*>(g.b) + (static_cast<size_t>(ew) * N + nv_pn0) * w_bytes +
                 (n - nv_pn0) * RB + c * 16;
    } else {
      b_src[q] = static_cast<const uint8_t*>(g.b) + (static_cast<size_t>(ew) * N + n) * w_bytes + c * 16;
    }
    b_dst[q] = B_OFF + qi * 1024;
    b_tail[q] = -((n - nv_pn0) * (RB / 2) + (c & (CPR / 2)) * 16);
  }

  // issue the direct loads of one K step into buffer buf.  Steps past the end
  // re-read the last step (that buffer is not read again); a chunk past the
  // FP8 K tail reads the in-range chunk 64 bytes earlier and is zeroed when
  // the fragments are formed.
  auto dma = [&](int step_in, uint8_t* buf, auto nt_c) {
    // weight loads carry the non-temporal cache-policy bit (aux bit 1) when
    // no other workgroup reads this weight panel
    constexpr int kWeightPolicy = decltype(nt_c)::value ? 2 : 0;
    const int step = min(step_in, n_steps - 1);
    const int kb = step * 128;                 // activation bytes before this step
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const uint8_t* p = a_src[q] + kb;
      if constexpr (FMT == kFP8) p = (kb + a_cof[q] >= a_bytes) ? p - 64 : p;
      __builtin_amdgcn_global_load_lds(p, (__attribute__((address_space(3))) void*)(buf + a_dst[q]),
                                       16, 0, 0);
    }
    const int wb = step * w_step;              // weight bytes before this step
    const bool tail = fp8_tail_step && step == n_steps - 1;
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const uint8_t* p = b_src[q] + wb;
      if constexpr (FMT == kFP8) p = tail ? p + b_tail[q] : p;
      __builtin_amdgcn_global_load_lds(p, (__attribute__((address_space(3))) void*)(buf + b_dst[q]),
                                       16, 0, kWeightPolicy);
    }
  };

  // row blocks dealt to wave rows in turn (as in grouped_gemm_kernel).  A
  // wave whose columns all lie past N (ragged last column tile) multiplies
  // nothing; it still issues its share of the loads and meets the barriers.
  const int live_blocks = (rows_valid + 31) >> 5;
  int ml_raw = (live_blocks - wm + WM - 1) / WM;
  ml_raw = ml_raw < 0 ? 0 : (ml_raw > MB ? MB : ml_raw);
  if (n0 + wn * WTN >= N) ml_raw = 0;
  const int ml = __builtin_amdgcn_readfirstlane(ml_raw);
  bool n_live[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) n_live[j] = n0 + wn * WTN + j * 32 < N;

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31;
  const int lk = lane >> 5;
  // byte offsets of this lane's rows inside a buffer, and their swizzles
  int a_row[MB], a_sw[MB], b_row[NB], b_sw[NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = (i * WM + wm) * 32 + lrow;
    a_row[i] = A_OFF + r * 128;
    a_sw[i] = lds_swz<128>(r);
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int r = wn * WTN + j * 32 + lrow;
    b_row[j] = B_OFF + r * RB;
    b_sw[j] = lds_swz<RB>(r);
  }

  using frag = bf16x8;
  // weight fragments of one lane for the 4 sub-steps of a step (expanded FP8)
  auto weight_frags = [&](const uint8_t* buf, int j, frag (&out)[4]) {
    if constexpr (FMT == kFP8X) {
      // 32 E4M3 codes at K 32 lk .. 32 lk + 31 -> bf16 (unit scale: exact)
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(buf + b_row[j] + (((2 * lk) ^ b_sw[j]) << 4));
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(buf + b_row[j] + (((2 * lk + 1) ^ b_sw[j]) << 4));
      const uint32_t w[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * s], 1.0f, false);
        const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * s], 1.0f, true);
        const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * s + 1], 1.0f, false);
        const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * s + 1], 1.0f, true);
        out[s] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
    }
  };

  auto compute = [&](const uint8_t* buf, int step, auto ml_c) {
    constexpr int ML = decltype(ml_c)::value;
    if constexpr (ML > 0) {
      if constexpr (FMT == kFP8) {
        // the second 64-byte half of the last step lies past K when K % 128 ==
        // 64: that half is skipped (its products would all be zero, and an
        // accumulator that starts at +0 stays unchanged by adding +0)
        const bool tail = (step * 128 + 64 >= a_bytes);
#pragma unroll
        for (int s = 0; s < 2; ++s) {  // 64 K per MFMA: chunks 4s + 2lk, +1
          if (s == 1 && tail) break;
          i32x8 af[ML], bfr[NB];
          const int c0 = s * 4 + lk * 2;
#pragma unroll
          for (int i = 0; i < ML; ++i) {
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(buf + a_row[i] + ((c0 ^ a_sw[i]) << 4));
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(buf + a_row[i] + (((c0 + 1) ^ a_sw[i]) << 4));
            af[i] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                          (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
          }
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(buf + b_row[j] + ((c0 ^ b_sw[j]) << 4));
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(buf + b_row[j] + (((c0 + 1) ^ b_sw[j]) << 4));
            bfr[j] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                           (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
          }
#pragma unroll
          for (int i = 0; i < ML; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  af[i], bfr[j], acc[i][j], 0, 0, 0, 127, 0, 127);
        }
      } else if constexpr (EXPAND) {
        frag bx[NB][4];
#pragma unroll
        for (int j = 0; j < NB; ++j) weight_frags(buf, j, bx[j]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {  // K 32 lk + 8 s .. + 8: activation chunk 4 lk + s
          const int c = lk * 4 + s;
          frag af[ML];
#pragma unroll
          for (int i = 0; i < ML; ++i)
            af[i] = *reinterpret_cast<const frag*>(buf + a_row[i] + ((c ^ a_sw[i]) << 4));
#pragma unroll
          for (int i = 0; i < ML; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bx[j][s], acc[i][j], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {  // 16 K per MFMA: chunk 2s + lk
          const int c = s * 2 + lk;
          bf16x8 af[ML], bfr[NB];
#pragma unroll
          for (int i = 0; i < ML; ++i)
            af[i] = *reinterpret_cast<const bf16x8*>(buf + a_row[i] + ((c ^ a_sw[i]) << 4));
#pragma unroll
          for (int j = 0; j < NB; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8*>(buf + b_row[j] + ((c ^ b_sw[j]) << 4));
#pragma unroll
          for (int i = 0; i < ML; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  // one K step: wait for this wave's loads of the step, meet, start the loads
  // NBUF - 1 steps ahead into the buffer everyone finished reading, multiply
  auto body = [&](int step, const uint8_t* cur, uint8_t* ahead, auto ml_c, auto nt_c) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NBUF - 2) * DPS));
    __asm__ volatile("s_barrier" ::: "memory");
    dma(step + NBUF - 1, ahead, nt_c);
    if (step < n_steps) compute(cur, step, ml_c);
  };
  auto main_loop = [&](auto ml_c, auto nt_c) {
    dma(0, lds0, nt_c);
    if constexpr (NBUF == 4) {
      dma(1, lds1, nt_c);
      dma(2, lds2, nt_c);
      for (int step = 0; step < n_steps; step += 4) {
        body(step, lds0, lds3, ml_c, nt_c);
        body(step + 1, lds1, lds0, ml_c, nt_c);
        body(step + 2, lds2, lds1, ml_c, nt_c);
        body(step + 3, lds3, lds2, ml_c, nt_c);
      }
    } else if constexpr (NBUF == 3) {
      dma(1, lds1, nt_c);
      for (int step = 0; step < n_steps; step += 3) {
        body(step, lds0, lds2, ml_c, nt_c);
        body(step + 1, lds1, lds0, ml_c, nt_c);
        body(step + 2, lds2, lds1, ml_c, nt_c);
      }
    } else {
      for (int step = 0; step < n_steps; step += 2) {
        body(step, lds0, lds1, ml_c, nt_c);
        body(step + 1, lds1, lds0, ml_c, nt_c);
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };
  static_assert(MB <= 4, "row blocks per wave");
  auto run = [&](auto nt_c) {
    switch (ml) {
      case 0: main_loop(std::integral_constant<int, 0>{}, nt_c); break;
      case 1: main_loop(std::integral_constant<int, (MB >= 1 ? 1 : MB)>{}, nt_c); break;
      case 2: main_loop(std::integral_constant<int, (MB >= 2 ? 2 : MB)>{}, nt_c); break;
      case 3: main_loop(std::integral_constant<int, (MB >= 3 ? 3 : MB)>{}, nt_c); break;
      default: main_loop(std::integral_constant<int, MB>{}, nt_c); break;
    }
  };
  // decode tiles: non-temporal weight loads when this workgroup is the
  // panel's only reader (the expert has one row tile), as in
  // grouped_gemm_kernel.  Prefill tiles keep one code path (a second one
  // costs registers: 132 VGPRs for the FP8 up tile, over the 128 that two
  // workgroups per CU allow).
  if constexpr (BM <= 32) {
    if (te == 1) run(std::true_type{});
    else run(std::false_type{});
  } else {
    run(std::false_type{});
  }

  // ---- epilogue (as in grouped_gemm_kernel)
  double scale = 1.0;
  if constexpr (FMT != kBF16) scale = static_cast<double>(g.a_s[0]) * static_cast<double>(g.b_s[e]);
  const float scale_f = static_cast<float>(scale);
  float local_max = 0.f;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if (i >= ml) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (!n_live[j]) continue;
      const int col = n0 + wn * WTN + j * 32 + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = (i * WM + wm) * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
        if (rl < rows_valid && col < N) {
          const size_t at = static_cast<size_t>(row0 + rl) * N + col;
          if constexpr (STAGE == 0) {
            // a = bf16(relu(h)^2), rounded once from the exact square of the
            // fp32 h (BF16: the accumulator itself)
            float h = acc[i][j][r];
            if constexpr (FMT != kBF16) h *= scale_f;
            const uint16_t b = relu_sq_bf16(h);
            static_cast<uint16_t*>(g.out)[at] = b;
            if constexpr (FMT != kBF16) local_max = fmaxf(local_max, bf16_to_f32(b));
          } else {
            const float gate = g.row_gate[row0 + rl];
            float o;
            if constexpr (FMT == kBF16) {
              o = acc[i][j][r] * gate;
            } else {
              o = acc[i][j][r] * (scale_f * gate);
            }
            static_cast<float*>(g.out)[at] = o;
          }
        }
      }
    }
  }
  if constexpr (STAGE == 0 && FMT != kBF16) block_amax_to_slots(local_max, g.amax);
}

// ---------------------------------------------------------------------------
// NVFP4 kernel (prefill and decode): weights straight into registers,
// activations through LDS.  In the bank's panel layout one K step (64
// elements) of 32 consecutive
// weight rows is 1 KB of codes and 128 bytes of block scales, contiguous, and
// exactly what one wave's MFMA fragments need: lane l takes row l % 32, codes
// of K [32 (l / 32), + 32) (16 bytes) and the row's 4 block scales.  So each
// wave loads its own 32 columns with one 16-byte and one 4-byte load per
// step, NBUF - 1 steps ahead in a register ring, and no weight byte passes
// through LDS.  LDS holds only the activation tile (BM rows of 128 bytes per
// step, direct global -> LDS loads, XOR-swizzled as in the kernel above), in
// NBUF buffers.  NW waves own 32 columns each, all BM rows (one wave row), so
// every weight block is expanded once; a wave reads its activation
// fragments of sub-step q + 1 while the MFMAs of sub-step q run.
template <int STAGE, int BM, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void grouped_gemm_nv_kernel(GemmArgs g) {
  static_assert(NBUF >= 2 && NBUF <= 4, "buffers");
  constexpr int BN = 32 * NW;
  constexpr int MB = BM / 32;                 // 32-row blocks per wave
  constexpr int NA = BM / 8;                  // activation loads per step (8 rows each)
  static_assert(NA % NW == 0 && MB <= 4, "tile");
  constexpr int QA = NA / NW;                 // activation loads per wave per step
  constexpr int ABUF = BM * 128;
  // one array per buffer: the compiler then knows that the direct loads into
  // one buffer do not write the buffer being read, and waits only for the
  // loads the reads need
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[ABUF];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[ABUF];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[NBUF >= 3 ? ABUF : 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[NBUF >= 4 ? ABUF : 1024];

  // ---- which tile (same order as the kernels above)
  const int n_ntiles = (g.N + BN - 1) / BN;
  const int total = g.tile_off[g.E] * n_ntiles;
  const int per_xcd = (total + 7) >> 3;
  const int local = blockIdx.x >> 3;
  if (local >= per_xcd) return;
  const int logical = (blockIdx.x & 7) * per_xcd + local;
  if (logical >= total) return;
  const int e = owner_expert(g.tile_off, g.E, n_ntiles, logical);
  const int te = g.tile_off[e + 1] - g.tile_off[e];
  const int loc = logical - g.tile_off[e] * n_ntiles;
  const int ntile = loc / te;
  const int mt = loc - ntile * te;
  const int row0 = g.offsets[e] + mt * BM;
  const int rows_valid = min(BM, g.offsets[e + 1] - row0);
  const int n0 = ntile * BN;
  const int ew = g.w_slot ? g.w_slot[e] : e;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = g.K, N = g.N;
  const int a_bytes = K * 2;                  // fp16 activation row bytes
  const int n_steps = K / 64;                 // K is a multiple of 64

  // ---- activation direct loads (fixed sources over K)
  const uint8_t* a_src[QA];
  int a_dst[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int qi = wave + q * NW;
    const int r = qi * 8 + (lane >> 3);
    const int c = (lane & 7) ^ lds_swz<128>(r);
    const int rr = min(r, rows_valid - 1);
    size_t src;
    if constexpr (STAGE == 0) {
      src = static_cast<size_t>(g.sorted_src[row0 + rr] / g.top_k);
    } else {
      src = static_cast<size_t>(row0 + rr);
    }
    a_src[q] = static_cast<const uint8_t*>(g.a) + src * a_bytes + c * 16;
    a_dst[q] = qi * 1024;
  }

  // ---- this lane's weight row in the panel layout (columns past N read the
  // last row; they are masked in the epilogue)
  const int lrow = lane & 31;
  const int lk = lane >> 5;
  const int wcol0 = n0 + wave * 32;
  const int n = min(wcol0 + lrow, N - 1);
  const int pn0 = n - n % kNvPanel;
  const int p_rows = nv_panel_rows(N, pn0 / kNvPanel);
  const uint8_t* b_code = static_cast<const uint8_t*>(g.b) +
                          (static_cast<size_t>(ew) * N + pn0) * (K / 2) + (n - pn0) * 32 + lk * 16;
  const uint8_t* b_scale = g.b_bs + (static_cast<size_t>(ew) * N + pn0) * (K / 16) + (n - pn0) * 4;
  const int code_step = p_rows * 32, scale_step = p_rows * 4;

  u32x4 bc[NBUF];
  uint32_t bsc[NBUF];

  // loads of step `step_in` (clamped: steps past the end re-read the last one)
  // (the global address goes through a named pointer: an arithmetic
  // expression as the builtin's first argument makes the host pass drop the
  // kernel's host stub without a diagnostic)
  // A wave that multiplies nothing (ML = 0: its columns lie past N) loads no
  // weights; its loads per step are then QA, not QA + 2, and the waits below
  // count exactly the loads issued (an unused load left to the compiler would
  // be removed and the count would be off).
  // NT: weights with the non-temporal cache policy (a weight panel that only
  // this workgroup reads, as in the kernels above).
  auto issue = [&](int step_in, uint8_t* buf, auto& codes, auto& scales, auto ml_c, auto nt_c) {
    constexpr int ML = decltype(ml_c)::value;
    constexpr bool NT = decltype(nt_c)::value;
    const int step = min(step_in, n_steps - 1);
    const int kb = step * 128;
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const uint8_t* p = a_src[q] + kb;
      __builtin_amdgcn_global_load_lds(p, (__attribute__((address_space(3))) void*)(buf + a_dst[q]),
                                       16, 0, 0);
    }
    if constexpr (ML > 0) {
      const u32x4* pc = reinterpret_cast<const u32x4*>(b_code + static_cast<size_t>(step) * code_step);
      const uint32_t* ps =
          reinterpret_cast<const uint32_t*>(b_scale + static_cast<size_t>(step) * scale_step);
      if constexpr (NT) {
        codes = __builtin_nontemporal_load(pc);
        scales = __builtin_nontemporal_load(ps);
      } else {
        codes = *pc;
        scales = *ps;
      }
    }
  };

  // live 32-row blocks; a wave whose columns all lie past N multiplies nothing
  const int live_blocks = (rows_valid + 31) >> 5;
  int ml_raw = live_blocks > MB ? MB : live_blocks;
  if (wcol0 >= N) ml_raw = 0;
  const int ml = __builtin_amdgcn_readfirstlane(ml_raw);

  f32x16 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  int a_row[MB], a_sw[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = i * 32 + lrow;
    a_row[i] = r * 128;
    a_sw[i] = lds_swz<128>(r);
  }

  // multiply one step: expand the lane's 32 codes (times their block scales)
  // into four fp16 fragments, then four sub-steps of ML MFMAs
  auto compute = [&](const uint8_t* buf, const u32x4 x, const uint32_t sc4, auto ml_c) {
    constexpr int ML = decltype(ml_c)::value;
    if constexpr (ML > 0) {
      const f16x2 scs = lk ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc4, 1.0f, true)
                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc4, 1.0f, false);
      f16x8 af[2][ML];
      auto rd = [&](int q, int slot) {
        const int c = lk * 4 + q;
#pragma unroll
        for (int i = 0; i < ML; ++i)
          af[slot][i] = *reinterpret_cast<const f16x8*>(buf + a_row[i] + ((c ^ a_sw[i]) << 4));
      };
      rd(0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q < 3) rd(q + 1, (q + 1) & 1);
        const _Float16 sc = q < 2 ? scs[0] : scs[1];
        const f16x2 s2 = {sc, sc};
        const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x[q], 1.0f, 0) * s2;
        const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x[q], 1.0f, 1) * s2;
        const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x[q], 1.0f, 2) * s2;
        const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x[q], 1.0f, 3) * s2;
        const f16x8 bfrag = f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
        for (int i = 0; i < ML; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[q & 1][i], bfrag, acc[i], 0, 0, 0);
      }
    }
  };

  // one K step: wait for this wave's loads of the step (activations into
  // LDS, weights into the ring), meet, start the loads NBUF - 1 steps ahead
  // into the buffer and ring slot everyone finished with, multiply
  uint8_t* const bufs[4] = {lds0, lds1, lds2, lds3};
  auto body = [&](int step, auto j_c, auto ml_c, auto nt_c) {
    constexpr int J = decltype(j_c)::value;
    constexpr int AHEAD = (J + NBUF - 1) % NBUF;
    constexpr int DPS = QA + (decltype(ml_c)::value > 0 ? 2 : 0);  // loads per step
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NBUF - 2) * DPS));
    __asm__ volatile("s_barrier" ::: "memory");
    issue(step + NBUF - 1, bufs[AHEAD], bc[AHEAD], bsc[AHEAD], ml_c, nt_c);
    if (step < n_steps) compute(bufs[J], bc[J], bsc[J], ml_c);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  auto main_loop = [&](auto ml_c, auto nt_c) {
    issue(0, lds0, bc[0], bsc[0], ml_c, nt_c);
    if constexpr (NBUF >= 3) issue(1, lds1, bc[1], bsc[1], ml_c, nt_c);
    if constexpr (NBUF >= 4) issue(2, lds2, bc[2], bsc[2], ml_c, nt_c);
    for (int step0 = 0; step0 < n_steps; step0 += NBUF) {
      body(step0, I0{}, ml_c, nt_c);
      body(step0 + 1, I1{}, ml_c, nt_c);
      if constexpr (NBUF >= 3) body(step0 + 2, I2{}, ml_c, nt_c);
      if constexpr (NBUF >= 4) body(step0 + 3, I3{}, ml_c, nt_c);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };
  auto run = [&](auto nt_c) {
    switch (ml) {
      case 0: main_loop(std::integral_constant<int, 0>{}, nt_c); break;
      case 1: main_loop(std::integral_constant<int, (MB >= 1 ? 1 : MB)>{}, nt_c); break;
      case 2: main_loop(std::integral_constant<int, (MB >= 2 ? 2 : MB)>{}, nt_c); break;
      case 3: main_loop(std::integral_constant<int, (MB >= 3 ? 3 : MB)>{}, nt_c); break;
      default: main_loop(std::integral_constant<int, MB>{}, nt_c); break;
    }
  };
  // decode tiles: non-temporal weight loads when this workgroup is the
  // panel's only reader (the expert has one row tile); prefill tiles keep one
  // code path
  if constexpr (BM <= 32) {
    if (te == 1) run(std::true_type{});
    else run(std::false_type{});
  } else {
    run(std::false_type{});
  }

  // ---- epilogue (as in the kernels above, one wave row)
  const float scale_f =
      static_cast<float>(static_cast<double>(g.a_s[0]) * static_cast<double>(g.b_s[e]));
  float local_max = 0.f;
  const int col = wcol0 + lrow;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if (i >= ml) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
      if (rl < rows_valid && col < N) {
        const size_t at = static_cast<size_t>(row0 + rl) * N + col;
        if constexpr (STAGE == 0) {
          const uint16_t b = relu_sq_bf16(acc[i][r] * scale_f);
          static_cast<uint16_t*>(g.out)[at] = b;
          local_max = fmaxf(local_max, bf16_to_f32(b));
        } else {
          const float gate = g.row_gate[row0 + rl];
          static_cast<float*>(g.out)[at] = acc[i][r] * (scale_f * gate);
        }
      }
    }
  }
  if constexpr (STAGE == 0) block_amax_to_slots(local_max, g.amax);
}

// One launch of a GEMM kernel over `blocks` workgroups (a multiple of the 8
// XCDs).  With timing events the launch goes through hipExtLaunchKernel, which
// stamps them with the kernel's own start and end; a launch with no tiles
// records both events back to back.
hipError_t dispatch(const void* kernel, long long blocks, int threads, const GemmArgs& g,
                    hipStream_t stream, const KernelEvents& ev) {
  const bool timed = ev.start || ev.stop;
  if (blocks <= 0) {
    hipError_t e = hipSuccess;
    if (ev.start) e = hipEventRecord(ev.start, stream);
    if (ev.stop && e == hipSuccess) e = hipEventRecord(ev.stop, stream);
    return e;
  }
  GemmArgs a = g;
  void* args[] = {&a};
  if (timed)
    return hipExtLaunchKernel(kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), args, 0,
                              stream, ev.start, ev.stop, 0);
  return hipLaunchKernel(kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), args, 0,
                         stream);
}

template <int FMT, int STAGE, int BM, int BN, int WM, int WN, int NBUF>
hipError_t launch_dma(const GemmArgs& g, hipStream_t stream, const KernelEvents& ev) {
  const int n_ntiles = (g.N + BN - 1) / BN;
  long long blocks = static_cast<long long>(g.max_tiles) * n_ntiles;
  blocks = (blocks + 7) / 8 * 8;
  return dispatch(reinterpret_cast<const void*>(
                      &grouped_gemm_dma_kernel<FMT, STAGE, BM, BN, WM, WN, NBUF>),
                  blocks, WM * WN * 64, g, stream, ev);
}

template <int STAGE, int BM, int NW, int NBUF>
hipError_t launch_nv(const GemmArgs& g, hipStream_t stream, const KernelEvents& ev) {
  const int n_ntiles = (g.N + 32 * NW - 1) / (32 * NW);
  long long blocks = static_cast<long long>(g.max_tiles) * n_ntiles;
  blocks = (blocks + 7) / 8 * 8;
  return dispatch(reinterpret_cast<const void*>(&grouped_gemm_nv_kernel<STAGE, BM, NW, NBUF>),
                  blocks, NW * 64, g, stream, ev);
}

template <int FMT, int STAGE, int BM, int BN, int WM, int WN>
hipError_t launch_one(const GemmArgs& g, hipStream_t stream, const KernelEvents& ev) {
  const int n_ntiles = (g.N + BN - 1) / BN;
  long long blocks = static_cast<long long>(g.max_tiles) * n_ntiles;
  blocks = (blocks + 7) / 8 * 8;
  return dispatch(reinterpret_cast<const void*>(&grouped_gemm_kernel<FMT, STAGE, BM, BN, WM, WN>),
                  blocks, WM * WN * 64, g, stream, ev);
}


template <int STAGE, int KS, int P>
hipError_t launch_rk(const GemmArgs& g, hipStream_t stream, const KernelEvents& ev) {
  const int n_ntiles = (g.N + 31) / 32;
  long long blocks = static_cast<long long>(g.max_tiles) * n_ntiles;
  blocks = (blocks + 7) / 8 * 8;
  return dispatch(reinterpret_cast<const void*>(&grouped_gemm_rk_kernel<STAGE, KS, P>), blocks,
                  KS * 64, g, stream, ev);
}

// Prefill tile of each format and projection (rows x columns, waves in M x N,
// LDS buffers), chosen by measurement on the 4096-token batch: 128 x 128
// tiles with eight 64 x 32 wave tiles and two buffers (two workgroups per CU)
// for BF16 and the FP8 down projection, 128 x 256 for the FP8 up projection
// (its weight rows are half as wide in LDS), all in the direct-load kernel.
template <int FMT, int STAGE>
struct PrefillTile {
  static constexpr int BM = 128, BN = 128, WM = 2, WN = 4, NBUF = 2;
};
template <>
struct PrefillTile<kFP8X, 0> {
  static constexpr int BM = 128, BN = 256, WM = 2, WN = 4, NBUF = 2;
};
// NVFP4 runs in grouped_gemm_nv_kernel: 128 x 256 tiles of eight 128 x 32
// wave tiles, activation buffers 2 (up) / 3 (down).  At 4096 tokens: up 308 ->
// 281 us and down 368 -> 299 us against the direct-load kernel's 128 x 128
// tiles (128 columns: 299 / 368 us; 256 columns with 3 buffers for up: 330 us,
// with 2 for down: 324 us; 128 columns with 3 / 4 buffers: 286 / 314 us up).
template <>
struct PrefillTile<kNVFP4, 0> {
  static constexpr int BM = 128, BN = 256, WM = 1, WN = 8, NBUF = 2;
};
template <>
struct PrefillTile<kNVFP4, 1> {
  static constexpr int BM = 128, BN = 256, WM = 1, WN = 8, NBUF = 3;
};

// decode batches: 32-row tiles, in the register-staged kernel (BF16, and the
// FP8 up projection with its codes expanded on the way into LDS) or the
// direct-load kernel with three LDS buffers (the FP8 down projection: 2-3 %
// faster than register staging at 4 and 64 tokens)
constexpr int kDecodeRows = 32;
constexpr int kDecodeMaxT = 512;
constexpr int kDecodeBuffers = 3;
// NVFP4 decode tiles run in grouped_gemm_nv_kernel (weights straight into
// registers, non-temporal for single-tile experts) with 4 activation buffers:
// T = 64 up 60.4 -> 53.3 us, down 56.5 -> 52.1 us against the direct-load
// kernel; T = 4 up 21.3 -> 18.1 us, down 16.1 -> 13.9 us (3 buffers: 19.8 /
// 15.8 us at T = 4, equal at T = 64; 2 buffers: equal at T = 64).
constexpr int kNvDecodeBuffers = 4;

// Below this many tokens the up projection touches so few experts that its
// workgroups cannot be spread evenly over the CUs (about 2.3 per CU at four
// tokens with 64-column tiles, so a third of the CUs stream 3 while the rest
// stream 2).  Narrower tiles give more, smaller work units: 32 columns and
// one wave for BF16, 64 columns and two waves for the expanded FP8 codes
// (measured fastest at four tokens; the down projection, with its wider N,
// is fastest with 128 columns).
constexpr int kNarrowUpMaxT = 16;

// BF16 decode of a single expert (the shared expert) over fewer 128-column
// tiles than this runs in the split-K kernel, 4 waves per 32 x 32 tile with
// 3 steps in flight each.  Shared expert of width 3712 in a BF16 block step:
// T = 64 0.359 -> 0.346 ms, T = 4 0.137 -> 0.110 ms (8 waves per tile, or 2
// or 4 steps in flight, measured within 1 % of this).  Routed batches keep
// the kernels above.
constexpr int kSmallGridTiles = 256;
constexpr int kSplitK = 4;
constexpr int kSplitDepth = 3;
inline bool small_decode_grid(const GemmArgs& g) {
  return g.E == 1 &&
         static_cast<long long>(g.max_tiles) * ((g.N + 127) / 128) < kSmallGridTiles;
}

template <int FMT, int STAGE>
hipError_t launch_fmt_stage(int T, const GemmArgs& g, hipStream_t stream, const KernelEvents& ev) {
  const bool decode = T < kDecodeMaxT;
  if constexpr (FMT == kNVFP4) {
    if (decode) return launch_nv<STAGE, kDecodeRows, 4, kNvDecodeBuffers>(g, stream, ev);
    using P = PrefillTile<FMT, STAGE>;
    return launch_nv<STAGE, P::BM, P::WN, P::NBUF>(g, stream, ev);
  } else {
    if constexpr (FMT == kFP8) {
      if (decode)
        return launch_dma<FMT, STAGE, kDecodeRows, 128, 1, 4, kDecodeBuffers>(g, stream, ev);
    } else {
      if constexpr (FMT == kBF16) {
        if (decode && small_decode_grid(g))
          return launch_rk<STAGE, kSplitK, kSplitDepth>(g, stream, ev);
      }
      if (STAGE == 0 && T < kNarrowUpMaxT) {
        if constexpr (FMT == kBF16)
          return launch_one<FMT, STAGE, kDecodeRows, 32, 1, 1>(g, stream, ev);
        return launch_one<FMT, STAGE, kDecodeRows, 64, 1, 2>(g, stream, ev);
      }
      if (decode) return launch_one<FMT, STAGE, kDecodeRows, 128, 1, 4>(g, stream, ev);
    }
    using P = PrefillTile<FMT, STAGE>;
    return launch_dma<FMT, STAGE, P::BM, P::BN, P::WM, P::WN, P::NBUF>(g, stream, ev);
  }
}

}  // namespace

GemmShape gemm_shape(int fmt, int stage, int T) {
  if (T < kDecodeMaxT) return GemmShape{kDecodeRows, 128};
  switch (fmt * 2 + stage) {
    case kBF16 * 2 + 0: return GemmShape{PrefillTile<kBF16, 0>::BM, PrefillTile<kBF16, 0>::BN};
    case kBF16 * 2 + 1: return GemmShape{PrefillTile<kBF16, 1>::BM, PrefillTile<kBF16, 1>::BN};
    case kFP8 * 2 + 0: return GemmShape{PrefillTile<kFP8X, 0>::BM, PrefillTile<kFP8X, 0>::BN};
    case kFP8 * 2 + 1: return GemmShape{PrefillTile<kFP8, 1>::BM, PrefillTile<kFP8, 1>::BN};
    case kNVFP4 * 2 + 0: return GemmShape{PrefillTile<kNVFP4, 0>::BM, PrefillTile<kNVFP4, 0>::BN};
    default: return GemmShape{PrefillTile<kNVFP4, 1>::BM, PrefillTile<kNVFP4, 1>::BN};
  }
}

hipError_t launch_gemm(int fmt, int stage, int T, const GemmArgs& g, hipStream_t stream,
                       const KernelEvents& ev) {
  switch (fmt * 2 + stage) {
    case kBF16 * 2 + 0: return launch_fmt_stage<kBF16, 0>(T, g, stream, ev);
    case kBF16 * 2 + 1: return launch_fmt_stage<kBF16, 1>(T, g, stream, ev);
    case kFP8 * 2 + 0: return launch_fmt_stage<kFP8X, 0>(T, g, stream, ev);
    case kFP8 * 2 + 1: return launch_fmt_stage<kFP8, 1>(T, g, stream, ev);
    case kNVFP4 * 2 + 0: return launch_fmt_stage<kNVFP4, 0>(T, g, stream, ev);
    case kNVFP4 * 2 + 1: return launch_fmt_stage<kNVFP4, 1>(T, g, stream, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
