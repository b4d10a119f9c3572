// Grouped expert GEMMs on MFMA (gfx950).
//
// The experts are ungated ReLU^2 FFNs: an up part 2688 -> 1856 and a down
// part 1856 -> 2688 (bloomery issue #967, section 2 "Checkpoint facts" and
// section 3 "Existing owners and gaps"); rows routed to one expert are
// multiplied together (grouped expert matmul, audio.cpp notes, section "CPU
// weight offload").
//
// One kernel template serves both projections and all three weight formats.
// A workgroup computes a BM x BN tile of one expert: BM sorted rows of that
// expert (from the permutation's device tile list) times BN output columns.
// Both operands are K-contiguous; each K step moves 128 bytes of every A and
// B row through double-buffered LDS (rows padded to 144 bytes, which keeps
// the 16-byte MFMA operand reads of 16 consecutive rows on distinct banks).
//   BF16 : v_mfma_f32_32x32x16_bf16, 64 K per step.
//   FP8  : v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales (E4M3 x
//          E4M3), 128 K per step; a 64-byte K tail (K = 1856 = 14*128 + 64)
//          is zero-filled in LDS rather than padded in HBM (zero padding of K
//          with matching zero activations leaves results unchanged: audio.cpp
//          notes, section "Q4_K, Q3_K and Q2_K expert profiles").
//   NVFP4: E2M1 codes and E4M3 block scales are expanded to bf16 while being
//          staged into LDS (code * block scale has at most 6 significant bits,
//          so the bf16 value is exact), then the BF16 MFMA; the two fp32 tensor
//          scales are applied in the epilogue.
// Epilogues: up writes bf16(relu(h)^2) (and the tensor amax for quantised
// formats); down writes fp32 gate * h per sorted row.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kStepBytes = 128;  // K bytes of each A/B row staged per step
constexpr int kLds = 144;        // padded LDS row stride in bytes

template <int FMT, int STAGE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_kernel(GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int MB = WTM / 32, NB = WTN / 32;  // 32x32 MFMA blocks per wave
  constexpr int A_CH = BM * 8 / NT;            // 16-byte A chunks per thread per step
  constexpr int B_CH = (FMT == kNVFP4) ? (BN * 2 / NT) : (BN * 8 / NT);
  constexpr int ESZ = (FMT == kFP8) ? 1 : 2;   // bytes per staged element
  static_assert(MB >= 1 && NB >= 1 && A_CH >= 1 && B_CH >= 1, "tile shape");
  static_assert((BM * 8) % NT == 0, "A chunks");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (BM + BN) * kLds];
  uint8_t* const As = lds;
  uint8_t* const Bs = lds + 2 * BM * kLds;

  // ---- which tile: blocks are dealt round-robin to the 8 XCDs; give each
  // XCD a contiguous run of logical tiles so the row tiles of one expert and
  // column tile (same weight panel) share that XCD's L2.
  const int nblk = gridDim.x;  // a multiple of 8
  const int logical = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int n_ntiles = (g.N + BN - 1) / BN;
  const int ntile = logical / g.max_tiles;
  const int mt = logical - ntile * g.max_tiles;
  if (ntile >= n_ntiles || mt >= *g.n_tiles) return;
  const int2 tile = g.tiles[mt];
  const int e = tile.x, row0 = tile.y;
  const int rows_valid = min(BM, g.offsets[e + 1] - row0);
  const int n0 = ntile * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int K = g.K, N = g.N;
  const int k_bytes = K * ESZ;
  const int n_steps = (k_bytes + kStepBytes - 1) / kStepBytes;

  // ---- per-thread global sources (fixed over K)
  const uint8_t* a_src[A_CH];
  int a_dst[A_CH], a_col[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * NT;
    const int r = c >> 3, cc = c & 7;
    const int rr = min(r, rows_valid - 1);
    size_t src;
    if constexpr (STAGE == 0) {
      src = static_cast<size_t>(g.sorted_src[row0 + rr] / g.top_k);
    } else {
      src = static_cast<size_t>(row0 + rr);
    }
    a_src[i] = static_cast<const uint8_t*>(g.a) + src * k_bytes + cc * 16;
    a_col[i] = cc * 16;
    a_dst[i] = r * kLds + cc * 16;
  }
  const uint8_t* b_src[B_CH];
  const uint8_t* s_src[B_CH];
  int b_dst[B_CH], b_col[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * NT;
    if constexpr (FMT == kNVFP4) {
      const int r = c >> 1, half = c & 1;
      const int n = min(n0 + r, N - 1);
      const size_t row = static_cast<size_t>(e) * N + n;
      b_src[i] = static_cast<const uint8_t*>(g.b) + row * (K / 2) + half * 16;
      s_src[i] = g.b_bs + row * (K / 16) + half * 2;
      b_dst[i] = r * kLds + half * 64;
      b_col[i] = 0;
    } else {
      const int r = c >> 3, cc = c & 7;
      const int n = min(n0 + r, N - 1);
      const size_t row = static_cast<size_t>(e) * N + n;
      b_src[i] = static_cast<const uint8_t*>(g.b) + row * k_bytes + cc * 16;
      s_src[i] = nullptr;
      b_dst[i] = r * kLds + cc * 16;
      b_col[i] = cc * 16;
    }
  }

  u32x4 a_reg[A_CH];
  u32x4 b_reg[B_CH];
  uint32_t s_reg[B_CH];

  auto load = [&](int step) {
    const int kb = step * kStepBytes;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      if (FMT == kFP8 && kb + a_col[i] >= k_bytes) {
        a_reg[i] = u32x4{0u, 0u, 0u, 0u};
      } else {
        a_reg[i] = *reinterpret_cast<const u32x4*>(a_src[i] + kb);
      }
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      if constexpr (FMT == kNVFP4) {
        b_reg[i] = *reinterpret_cast<const u32x4*>(b_src[i] + step * 32);
        s_reg[i] = *reinterpret_cast<const uint16_t*>(s_src[i] + step * 4);
      } else {
        if (FMT == kFP8 && kb + b_col[i] >= k_bytes) {
          b_reg[i] = u32x4{0u, 0u, 0u, 0u};
        } else {
          b_reg[i] = *reinterpret_cast<const u32x4*>(b_src[i] + kb);
        }
      }
    }
  };

  auto store = [&](int buf) {
    uint8_t* A = As + buf * BM * kLds;
    uint8_t* B = Bs + buf * BN * kLds;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) *reinterpret_cast<u32x4*>(A + a_dst[i]) = a_reg[i];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      if constexpr (FMT == kNVFP4) {
        // 32 E2M1 codes (element 2j in the low nibble of byte j), two block scales
        const float sc0 = e4m3_decode(s_reg[i] & 0xffu);
        const float sc1 = e4m3_decode((s_reg[i] >> 8) & 0xffu);
        uint32_t outw[16];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t word = b_reg[i][w];
          const float sc = w < 2 ? sc0 : sc1;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const uint32_t byte = (word >> (8 * bb)) & 0xffu;
            const float v0 = e2m1_decode(byte & 15u) * sc;  // exact
            const float v1 = e2m1_decode(byte >> 4) * sc;
            outw[w * 4 + bb] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xffff0000u);
          }
        }
        u32x4* dst = reinterpret_cast<u32x4*>(B + b_dst[i]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dst[q] = u32x4{outw[4 * q], outw[4 * q + 1], outw[4 * q + 2], outw[4 * q + 3]};
      } else {
        *reinterpret_cast<u32x4*>(B + b_dst[i]) = b_reg[i];
      }
    }
  };

  // ---- which MFMA blocks of this wave hold live rows / columns
  bool m_live[MB], n_live[NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) m_live[i] = wm * WTM + i * 32 < rows_valid;
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

  auto compute = [&](int buf) {
    const uint8_t* A = As + buf * BM * kLds;
    const uint8_t* B = Bs + buf * BN * kLds;
    if constexpr (FMT == kFP8) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {  // 64 K per MFMA
        i32x8 af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const uint8_t* p = A + (wm * WTM + i * 32 + lrow) * kLds + s * 64 + lk * 32;
          const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
          af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const uint8_t* p = B + (wn * WTN + j * 32 + lrow) * kLds + s * 64 + lk * 32;
          const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
          bfr[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            if (m_live[i] && n_live[j])
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  af[i], bfr[j], acc[i][j], 0, 0, 0, 127, 0, 127);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {  // 16 K per MFMA
        bf16x8 af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(
              A + (wm * WTM + i * 32 + lrow) * kLds + s * 32 + lk * 16);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8*>(
              B + (wn * WTN + j * 32 + lrow) * kLds + s * 32 + lk * 16);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            if (m_live[i] && n_live[j])
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // ---- main loop: one barrier per K step (double-buffered LDS)
  load(0);
  store(0);
  __syncthreads();
  for (int step = 0; step < n_steps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < n_steps;
    if (more) load(step + 1);
    compute(buf);
    if (more) store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  32x32 f32 result: lane holds column lane%32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
  // scales of the quantised formats: s_act * s_weight, exact in double
  double scale = 1.0;
  if constexpr (FMT != kBF16) scale = static_cast<double>(g.a_s[0]) * static_cast<double>(g.b_s[e]);
  float local_max = 0.f;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if (!m_live[i]) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (!n_live[j]) continue;
      const int col = n0 + wn * WTN + j * 32 + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm * WTM + i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
        if (rl < rows_valid && col < N) {
          const size_t at = static_cast<size_t>(row0 + rl) * N + col;
          if constexpr (STAGE == 0) {
            // a = bf16(relu(h)^2): h^2 is exact in double, so a is rounded once
            double h = static_cast<double>(acc[i][j][r]);
            if constexpr (FMT != kBF16) h *= scale;
            const uint16_t b = h > 0.0 ? f64_to_bf16(h * h) : static_cast<uint16_t>(0);
            static_cast<uint16_t*>(g.out)[at] = b;
            if constexpr (FMT != kBF16) local_max = fmaxf(local_max, bf16_to_f32(b));
          } else {
            const float gate = g.row_gate[row0 + rl];
            float o;
            if constexpr (FMT == kBF16) {
              o = acc[i][j][r] * gate;
            } else {
              o = static_cast<float>(static_cast<double>(acc[i][j][r]) * scale * gate);
            }
            static_cast<float*>(g.out)[at] = o;
          }
        }
      }
    }
  }
  if constexpr (STAGE == 0 && FMT != kBF16) {
    local_max = wave_max(local_max);
    if (lane == 0) atomic_max_nonneg(g.amax, local_max);
  }
}

template <int FMT, int STAGE, int BM, int BN, int WM, int WN>
hipError_t launch_one(const GemmArgs& g, hipStream_t stream) {
  const int n_ntiles = (g.N + BN - 1) / BN;
  long long blocks = static_cast<long long>(g.max_tiles) * n_ntiles;
  blocks = (blocks + 7) / 8 * 8;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<FMT, STAGE, BM, BN, WM, WN>), dim3(blocks),
                     dim3(WM * WN * 64), 0, stream, g);
  return hipGetLastError();
}

template <int FMT, int STAGE>
hipError_t launch_fmt_stage(int T, const GemmArgs& g, hipStream_t stream) {
  const GemmShape s = gemm_shape(FMT, STAGE, T);
  if (s.bm == 32) return launch_one<FMT, STAGE, 32, 128, 1, 4>(g, stream);
  return launch_one<FMT, STAGE, 128, 128, 2, 2>(g, stream);
}

}  // namespace

GemmShape gemm_shape(int /*fmt*/, int /*stage*/, int T) {
  if (T < 512) return GemmShape{32, 128};
  return GemmShape{128, 128};
}

hipError_t launch_gemm(int fmt, int stage, int T, const GemmArgs& g, hipStream_t stream) {
  switch (fmt * 2 + stage) {
    case kBF16 * 2 + 0: return launch_fmt_stage<kBF16, 0>(T, g, stream);
    case kBF16 * 2 + 1: return launch_fmt_stage<kBF16, 1>(T, g, stream);
    case kFP8 * 2 + 0: return launch_fmt_stage<kFP8, 0>(T, g, stream);
    case kFP8 * 2 + 1: return launch_fmt_stage<kFP8, 1>(T, g, stream);
    case kNVFP4 * 2 + 0: return launch_fmt_stage<kNVFP4, 0>(T, g, stream);
    case kNVFP4 * 2 + 1: return launch_fmt_stage<kNVFP4, 1>(T, g, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
