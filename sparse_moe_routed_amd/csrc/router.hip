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
// router_logits_kernel (T <= 256) and router_logits_lds_kernel (larger
// batches) write partial logits of S slices of K to the workspace as [S, T, E]
// fp32; more slices spread small batches over more CUs.
// router_topk_kernel: one wave per token sums the S partials in order (all S
// loads issued together), adds the bias and takes k rounds of wave-wide
// maximum (DPP reductions, ties to the lower index), then writes the
// renormalised softmax gates.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kTokPerWave = 16;
constexpr int kWavesPerWg = 4;
constexpr int kTokPerWg = kTokPerWave * kWavesPerWg;
constexpr int kMaxE = 256;
constexpr int kMaxSlices = 12;  // router_k_slices never returns more

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

// Small batches: the 4 waves of a workgroup take 4 blocks of 16 tokens against
// one 16-expert block over one K slice, loading MFMA fragments straight from
// global memory with several K steps in flight (few tokens: latency-bound).
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wp,
                                                            int T, int H, int E, int S,
                                                            float* __restrict__ part) {
  constexpr int U = 4;  // K steps of loads in flight
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kTokPerWg + wave * kTokPerWave;
  const int eb = blockIdx.y;
  if (t0 >= T || eb * 16 >= E) return;  // no barriers in this kernel
  const int s = blockIdx.z;
  const int row = lane & 15;       // MFMA row (token) / column (expert) of this lane
  const int kq = (lane >> 4) * 8;  // this lane's 8-wide K slice inside a 32-K step
  const int kbeg = s * (H / S), kend = kbeg + H / S;
  const size_t n = static_cast<size_t>(E) * H;
  const uint16_t* xrow = x + static_cast<size_t>(min(t0 + row, T - 1)) * H + kq;
  const uint16_t* w_hi = wp + static_cast<size_t>(eb * 16 + row) * H + kq;
  const uint16_t* w_mid = w_hi + n;
  const uint16_t* w_lo = w_hi + 2 * n;

  f32x4 acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = kbeg; k0 < kend; k0 += U * 32) {
    bf16x8 a[U], bh[U], bm[U], bl[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // issue the loads of U K steps first
      const int kk = k0 + u * 32;
      if (kk < kend) {
        a[u] = *reinterpret_cast<const bf16x8*>(xrow + kk);
        bh[u] = *reinterpret_cast<const bf16x8*>(w_hi + kk);
        bm[u] = *reinterpret_cast<const bf16x8*>(w_mid + kk);
        bl[u] = *reinterpret_cast<const bf16x8*>(w_lo + kk);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u * 32 >= kend) break;
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bl[u], acc[u], 0, 0, 0);
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bm[u], acc[u], 0, 0, 0);
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bh[u], acc[u], 0, 0, 0);
    }
  }
  // 16x16 f32 result: lane holds column (expert) lane%16, rows 4*(lane/16)+r
  const int e = eb * 16 + row;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + (lane >> 4) * 4 + r;
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) v += acc[u][r];
    if (t < T) part[(static_cast<size_t>(s) * T + t) * E + e] = v;
  }
}

// Large batches: a workgroup takes 64 tokens x kLE experts over one K slice.
// Each 32-element K step stages the token tile (64 rows) and the three router
// parts (3 x kLE rows) in LDS with coalesced 16-byte loads, one step of
// register prefetch and double-buffered LDS; wave w multiplies all 64 tokens
// against experts 32w .. 32w + 31 out of LDS.  (Loading MFMA fragments
// straight from global memory touches 16 rows per instruction, which runs at
// a fraction of the coalesced rate.)
constexpr int kLE = 128;                // experts per workgroup
constexpr int kLRow = 80;               // LDS row stride: 64 data bytes + 16 pad
constexpr int kLRows = 64 + 3 * kLE;    // token rows + router rows per buffer
constexpr int kLChunks = kLRows * 4;    // 16-byte chunks per step
constexpr int kLPer = (kLChunks + 255) / 256;

__global__ __launch_bounds__(256) void router_logits_lds_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ wp,
                                                                int T, int H, int E, int S,
                                                                float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kLRows * kLRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * 64;
  const int s = blockIdx.y;
  const int e0 = blockIdx.z * kLE;
  const int kbeg = s * (H / S);
  const int n_steps = (H / S) / 32;
  const size_t n = static_cast<size_t>(E) * H;

  // this thread's chunks: row r (token rows first, then lo / mid / hi router
  // rows of the workgroup's experts), 16-byte piece q of the row's 64 bytes
  const uint16_t* src[kLPer];
  int dst[kLPer];
#pragma unroll
  for (int i = 0; i < kLPer; ++i) {
    const int c = min(tid + i * 256, kLChunks - 1);
    const int r = c >> 2, q = c & 3;
    if (r < 64) {
      src[i] = x + static_cast<size_t>(min(t0 + r, T - 1)) * H + kbeg + q * 8;
    } else {
      const int rr = r - 64, p = rr / kLE;
      const int e = min(e0 + rr % kLE, E - 1);
      // part order in LDS: lo, mid, hi (the accumulation order below)
      src[i] = wp + static_cast<size_t>(2 - p) * n + static_cast<size_t>(e) * H + kbeg + q * 8;
    }
    dst[i] = r * kLRow + q * 16;
  }
  u32x4 reg[kLPer];
  auto load = [&](int step) {
    const int k = min(step, n_steps - 1) * 32;
#pragma unroll
    for (int i = 0; i < kLPer; ++i) reg[i] = *reinterpret_cast<const u32x4*>(src[i] + k);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLPer; ++i) *reinterpret_cast<u32x4*>(&lds[buf][dst[i]]) = reg[i];
  };

  f32x4 acc[4][2];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int row = lane & 15;
  const int kq = (lane >> 4) * 16;  // byte offset of this lane's 8 K values
  auto compute = [&](int buf) {
    const uint8_t* L = lds[buf];
    bf16x8 a[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      a[b] = *reinterpret_cast<const bf16x8*>(L + (b * 16 + row) * kLRow + kq);
#pragma unroll
    for (int p = 0; p < 3; ++p) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 w = *reinterpret_cast<const bf16x8*>(
            L + (64 + p * kLE + wave * 32 + j * 16 + row) * kLRow + kq);
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[b], w, acc[b][j], 0, 0, 0);
      }
    }
  };

  load(0);
  store(0);
  load(1);
  __syncthreads();
  for (int step = 0; step < n_steps; ++step) {
    compute(step & 1);
    store((step + 1) & 1);
    load(step + 2);
    __syncthreads();
  }

  // 16x16 f32 result: lane holds column (expert) lane%16, rows 4*(lane/16)+r
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + wave * 32 + j * 16 + row;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + b * 16 + (lane >> 4) * 4 + r;
        if (t < T && e < E) part[(static_cast<size_t>(s) * T + t) * E + e] = acc[b][j][r];
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
// maps above 0, which marks an empty slot).  -0 and +0 compare equal as
// floats, so -0 is first made +0 (x + 0 is +0 for x = -0 under round to
// nearest) and both get one key: a tie between them goes to the lower index.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave per token: lane l holds experts l + 64 i.  Each of the k rounds
// takes the largest key over the wave, then the lowest expert index holding
// it (ballots over the slots in index order), and retires that expert.
// Gates: z_j = exp(l_j - l_0), summed in slot order, g_j = z_j / sum.
// MAXS >= S bounds the unrolled slice loads; slices past S read slice S - 1
// again and add +0 (the running sum starts at +0, so the result is the same
// as summing exactly S terms).
template <int MAXS>
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
      float p[MAXS];
#pragma unroll
      for (int s = 0; s < MAXS; ++s)
        p[s] = part[(static_cast<size_t>(min(s, S - 1)) * T + t) * E + e];
      const float b = bias ? bias[e] : 0.f;
      float l = 0.f;
#pragma unroll
      for (int s = 0; s < MAXS; ++s) l += s < S ? p[s] : 0.f;
      v[i] = l + b;
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
  int S = T <= 256 ? kMaxSlices : 4;
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
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, stream, x, w_packed, T, H, E, S,
                       part);
  } else {
    const dim3 grid((T + 63) / 64, S, (E + kLE - 1) / kLE);
    hipLaunchKernelGGL(router_logits_lds_kernel, grid, dim3(256), 0, stream, x, w_packed, T, H, E,
                       S, part);
  }
  const dim3 tgrid((T + kWavesPerWg - 1) / kWavesPerWg);
  if (S <= 4)
    hipLaunchKernelGGL(router_topk_kernel<4>, tgrid, dim3(256), 0, stream, part, bias, T, E, S, k,
                       ids, gates);
  else
    hipLaunchKernelGGL(router_topk_kernel<kMaxSlices>, tgrid, dim3(256), 0, stream, part, bias, T,
                       E, S, k, ids, gates);
  return hipGetLastError();
}

}  // namespace moe
