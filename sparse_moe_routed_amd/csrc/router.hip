// Router: fp32 logits of bf16 tokens against an fp32 router matrix, then
// top-k selection and renormalised softmax gates.
//
// Routing is top-6 over 128 experts (bloomery issue #967, section 2
// "Checkpoint facts") and is a formula of its own, separate from expert
// execution (audio.cpp notes "NVIDIA Nemotron 3.5 Transcribe", section "CPU
// weight offload").
//
// The logits are a dense [T, H] x [H, E] contraction, so they run on MFMA:
// each fp32 router weight w is split exactly into three bf16 parts
// (hi + mid + lo == w), and x is bf16, so every product x * part is exact in
// the fp32 accumulator of v_mfma_f32_16x16x32_bf16.  A workgroup owns 16
// tokens and all experts; its logits stay in LDS for the selection.  Its 16
// waves split the work as 8 expert blocks x 2 halves of K, and each wave keeps
// four K steps of loads in flight (the router matrix is re-read from L2 by
// every workgroup, so the loop is latency-bound, not bandwidth-bound).
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kTokTile = 16;   // tokens per workgroup (MFMA M)
constexpr int kRouterThreads = 1024;
constexpr int kKParts = 2;       // K halves per expert block
constexpr int kEBlkPar = 8;      // expert blocks processed side by side
constexpr int kMaxE = 256;

// exact split of an fp32 value into three bf16 values (truncations; the
// residual after two truncations has at most 8 significant bits)
__device__ __forceinline__ void split3(float w, __bf16& hi, __bf16& mid, __bf16& lo) {
  const uint32_t u = __float_as_uint(w);
  const float h = __uint_as_float(u & 0xffff0000u);
  const float r1 = w - h;
  const float m = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
  const float r2 = r1 - m;
  hi = __builtin_bit_cast(__bf16, static_cast<uint16_t>(u >> 16));
  mid = __builtin_bit_cast(__bf16, static_cast<uint16_t>(__float_as_uint(m) >> 16));
  lo = __builtin_bit_cast(__bf16, f32_to_bf16(r2));
}

__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w,
    const float* __restrict__ bias, int T, int H, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ gates) {
  __shared__ float logits[kKParts][kTokTile][kMaxE + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kTokTile;
  const int row = lane & 15;         // MFMA row (token) / column (expert) of this lane
  const int kq = (lane >> 4) * 8;    // this lane's 8-wide K slice inside a 32-K step
  const int tok = min(t0 + row, T - 1);
  const uint16_t* xrow = x + static_cast<size_t>(tok) * H + kq;
  const int n_eblk = E / 16;
  const int kp = wave / kEBlkPar;
  const int kbeg = kp * (H / kKParts), kend = kbeg + H / kKParts;

  for (int eb = wave % kEBlkPar; eb < n_eblk; eb += kEBlkPar) {
    const float* wrow = w + static_cast<size_t>(eb * 16 + row) * H + kq;
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = kbeg; k0 < kend; k0 += 4 * 32) {
      bf16x8 a[4];
      f32x4 w0[4], w1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // issue the loads of four K steps first
        const int kk = k0 + u * 32;
        if (kk < kend) {
          a[u] = *reinterpret_cast<const bf16x8*>(xrow + kk);
          w0[u] = *reinterpret_cast<const f32x4*>(wrow + kk);
          w1[u] = *reinterpret_cast<const f32x4*>(wrow + kk + 4);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (k0 + u * 32 >= kend) break;
        bf16x8 bh, bm, bl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __bf16 h0, m0, l0, h1, m1, l1;
          split3(w0[u][i], h0, m0, l0);
          split3(w1[u][i], h1, m1, l1);
          bh[i] = h0; bm[i] = m0; bl[i] = l0;
          bh[i + 4] = h1; bm[i + 4] = m1; bl[i + 4] = l1;
        }
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bl, acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bm, acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bh, acc[u], 0, 0, 0);
      }
    }
    // 16x16 f32 result: lane holds column (expert) lane%16, rows 4*(lane/16)+r
    const int e = eb * 16 + row;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      logits[kp][(lane >> 4) * 4 + r][e] = (acc[0][r] + acc[1][r]) + (acc[2][r] + acc[3][r]);
  }
  __syncthreads();

  // top-k: one token per wave; a lane holds experts lane + 64 i
  for (int tt = wave; tt < kTokTile; tt += kRouterThreads / 64) {
    const int t = t0 + tt;
    if (t >= T) break;
    float v[kMaxE / 64];
#pragma unroll
    for (int i = 0; i < kMaxE / 64; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? (logits[0][tt][e] + logits[1][tt][e]) + (bias ? bias[e] : 0.f) : -INFINITY;
    }
    float sel_v[8];
    int sel_i[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sel_v[j] = 0.f;
      sel_i[j] = 0;
      if (j >= k) continue;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kMaxE / 64; ++i) {
        const int e = lane + 64 * i;
        if (e < E && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      sel_v[j] = bv;
      sel_i[j] = bi;
#pragma unroll
      for (int i = 0; i < kMaxE / 64; ++i)
        if (lane + 64 * i == bi) v[i] = -INFINITY;  // remove the winner
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
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const float* w, const float* bias, int T,
                         int H, int E, int k, int32_t* ids, float* gates,
                         hipStream_t stream) {
  const int blocks = (T + kTokTile - 1) / kTokTile;
  hipLaunchKernelGGL(router_topk_kernel, dim3(blocks), dim3(kRouterThreads), 0, stream,
                     x, w, bias, T, H, E, k, ids, gates);
  return hipGetLastError();
}

}  // namespace moe
