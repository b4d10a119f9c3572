// Router: fp32 logits of bf16 tokens against an fp32 router matrix, then
// top-k selection and renormalised softmax gates.
//
// Routing is top-6 over 128 experts (bloomery issue #967, section 2
// "Checkpoint facts") and is a formula of its own, separate from expert
// execution (audio.cpp notes "NVIDIA Nemotron 3.5 Transcribe", section "CPU
// weight offload").
//
// The logits are a dense [T, H] x [H, E] contraction, so they run on MFMA.
// The fp32 router matrix is packed once (router_pack_kernel) into three bf16
// matrices with w == hi + mid + lo exactly; x is bf16, so every product
// x * part is exact in the fp32 accumulator of v_mfma_f32_16x16x32_bf16 and
// the logits carry only fp32 summation error.
//
// router_logits_kernel: a workgroup computes 64 tokens against 16 (small
// batches) or 64 experts over one of S slices of K (S > 1 spreads small
// batches over more CUs); waves keep several K steps of loads in flight.
// Partial logits go to the workspace as [S, T, E] fp32.
// router_topk_kernel: one wave per token sums the S partials in order, adds
// the bias and takes k rounds of wave-wide maximum (DPP reductions, ties to
// the lower index), then writes the renormalised softmax gates.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kTokPerWave = 16;
constexpr int kWavesPerWg = 4;
constexpr int kTokPerWg = kTokPerWave * kWavesPerWg;
constexpr int kMaxE = 256;

__global__ __launch_bounds__(256) void router_pack_kernel(const float* __restrict__ w, size_t n,
                                                          uint16_t* __restrict__ packed) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * 256) {
    const float v = w[i];
    const uint32_t u = __float_as_uint(v);
    const float hi = __uint_as_float(u & 0xffff0000u);  // truncation: exact residual
    const float r1 = v - hi;
    const float mid = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
    const float r2 = r1 - mid;  // at most 8 significant bits: exact in bf16
    packed[i] = static_cast<uint16_t>(u >> 16);
    packed[n + i] = static_cast<uint16_t>(__float_as_uint(mid) >> 16);
    packed[2 * n + i] = f32_to_bf16(r2);
  }
}

// TB = 16-token row blocks per wave.  TB == 1 (small batches): the 4 waves
// take 4 row blocks of one 16-expert block.  TB == 4: each wave takes all 64
// tokens of the workgroup against its own 16-expert block, reusing every
// router fragment for 4 MFMA row blocks (less L2 traffic per logit).
template <int TB>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wp,
                                                            int T, int H, int E, int S,
                                                            float* __restrict__ part) {
  constexpr int U = TB == 1 ? 4 : 2;  // K steps of loads in flight
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kTokPerWg + (TB == 1 ? wave * kTokPerWave : 0);
  const int eb = TB == 1 ? blockIdx.y : blockIdx.y * kWavesPerWg + wave;
  if (t0 >= T || eb * 16 >= E) return;  // no barriers in this kernel
  const int s = blockIdx.z;
  const int row = lane & 15;       // MFMA row (token) / column (expert) of this lane
  const int kq = (lane >> 4) * 8;  // this lane's 8-wide K slice inside a 32-K step
  const int kbeg = s * (H / S), kend = kbeg + H / S;
  const size_t n = static_cast<size_t>(E) * H;
  const uint16_t* xrow[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b)
    xrow[b] = x + static_cast<size_t>(min(t0 + b * 16 + row, T - 1)) * H + kq;
  const uint16_t* w_hi = wp + static_cast<size_t>(eb * 16 + row) * H + kq;
  const uint16_t* w_mid = w_hi + n;
  const uint16_t* w_lo = w_hi + 2 * n;

  f32x4 acc[TB][U];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int u = 0; u < U; ++u) acc[b][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = kbeg; k0 < kend; k0 += U * 32) {
    bf16x8 a[U][TB], bh[U], bm[U], bl[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // issue the loads of U K steps first
      const int kk = k0 + u * 32;
      if (kk < kend) {
#pragma unroll
        for (int b = 0; b < TB; ++b) a[u][b] = *reinterpret_cast<const bf16x8*>(xrow[b] + kk);
        bh[u] = *reinterpret_cast<const bf16x8*>(w_hi + kk);
        bm[u] = *reinterpret_cast<const bf16x8*>(w_mid + kk);
        bl[u] = *reinterpret_cast<const bf16x8*>(w_lo + kk);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u * 32 >= kend) break;
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        acc[b][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][b], bl[u], acc[b][u], 0, 0, 0);
        acc[b][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][b], bm[u], acc[b][u], 0, 0, 0);
        acc[b][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][b], bh[u], acc[b][u], 0, 0, 0);
      }
    }
  }
  // 16x16 f32 result: lane holds column (expert) lane%16, rows 4*(lane/16)+r
  const int e = eb * 16 + row;
#pragma unroll
  for (int b = 0; b < TB; ++b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + b * 16 + (lane >> 4) * 4 + r;
      float v = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) v += acc[b][u][r];
      if (t < T) part[(static_cast<size_t>(s) * T + t) * E + e] = v;
    }
  }
}

// Largest 32-bit unsigned value over the wave, in every lane.  DPP row shifts
// reduce each 16-lane row into its lane 15, two row broadcasts combine the
// rows into lane 63; zero (the identity) fills lanes a shift leaves empty.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// order-preserving unsigned key of a float (larger float -> larger key; -inf
// maps above 0, which marks an empty slot)
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave per token: lane l holds experts l + 64 i.  Each of the k rounds
// takes the largest key over the wave, then the lowest expert index holding
// it (ballots over the slots in index order), and retires that expert.
// Gates: z_j = exp(l_j - l_0), summed in slot order, g_j = z_j / sum.
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ part,
                                                          const float* __restrict__ bias, int T,
                                                          int E, int S, int k,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWavesPerWg + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves; no barriers below
  float v[kMaxE / 64];
  uint32_t key[kMaxE / 64];
#pragma unroll
  for (int i = 0; i < kMaxE / 64; ++i) {
    const int e = lane + 64 * i;
    v[i] = -INFINITY;
    key[i] = 0u;
    if (e < E) {
      float l = 0.f;
      for (int s = 0; s < S; ++s) l += part[(static_cast<size_t>(s) * T + t) * E + e];
      v[i] = l + (bias ? bias[e] : 0.f);
      key[i] = float_key(v[i]);
    }
  }
  float sel_v[8];
  int sel_i[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sel_v[j] = 0.f;
    sel_i[j] = 0;
    if (j >= k) continue;
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < kMaxE / 64; ++i) m = max(m, key[i]);
    const uint32_t best = wave_umax(m);
    int win = -1;
#pragma unroll
    for (int i = 0; i < kMaxE / 64; ++i) {
      const uint64_t b = __ballot(key[i] == best && key[i] != 0u);
      if (win < 0 && b) win = 64 * i + __ffsll(static_cast<unsigned long long>(b)) - 1;
    }
    // the winner's logit, from the lane that holds it
    float wv = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxE / 64; ++i)
      if (lane + 64 * i == win) {
        wv = v[i];
        key[i] = 0u;
      }
    sel_v[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wv), win & 63));
    sel_i[j] = win;
  }
  if (lane == 0) {
    const float m = sel_v[0];
    float z[8];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      z[j] = j < k ? expf(sel_v[j] - m) : 0.f;
      sum += z[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        ids[static_cast<size_t>(t) * k + j] = sel_i[j];
        gates[static_cast<size_t>(t) * k + j] = z[j] / sum;
      }
    }
  }
}

}  // namespace

// K slices: each wave's K loop is a chain of L2 round trips, so the router
// splits K into slices of whole 32-element MFMA steps: up to 12 for small
// batches (few token blocks to spread over the CUs), up to 4 otherwise.
int router_k_slices(int T, int H) {
  const int steps = H / 32;
  int S = T <= 256 ? 12 : 4;
  while (S > 1 && steps % S) --S;
  return S;
}

hipError_t launch_router_pack(const float* w, int E, int H, uint16_t* packed, hipStream_t stream) {
  const size_t n = static_cast<size_t>(E) * H;
  size_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(router_pack_kernel, dim3(static_cast<unsigned>(g)), dim3(256), 0, stream, w,
                     n, packed);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const uint16_t* w_packed, const float* bias, int T,
                         int H, int E, int k, float* part, int32_t* ids, float* gates,
                         hipStream_t stream) {
  const int S = router_k_slices(T, H);
  if (T <= 256) {
    const dim3 grid((T + kTokPerWg - 1) / kTokPerWg, E / 16, S);
    hipLaunchKernelGGL(router_logits_kernel<1>, grid, dim3(256), 0, stream, x, w_packed, T, H, E,
                       S, part);
  } else {
    const dim3 grid((T + kTokPerWg - 1) / kTokPerWg, (E / 16 + kWavesPerWg - 1) / kWavesPerWg, S);
    hipLaunchKernelGGL(router_logits_kernel<4>, grid, dim3(256), 0, stream, x, w_packed, T, H, E,
                       S, part);
  }
  hipLaunchKernelGGL(router_topk_kernel, dim3((T + kWavesPerWg - 1) / kWavesPerWg), dim3(256), 0,
                     stream, part, bias, T, E, S, k, ids, gates);
  return hipGetLastError();
}

}  // namespace moe
