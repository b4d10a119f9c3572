// Gate-weighted combine of the per-slot expert rows, plus the stacked-path
// helpers (weightless RMS pre-norm and residual add).
//
// The down GEMM has already multiplied each sorted row by its gate, so the
// combine gathers the k rows of a token in slot order j = 0..k-1 and adds
// them in fp32: a deterministic gather, no atomics.  The routing weights are
// their own formula (audio.cpp notes "NVIDIA Nemotron 3.5 Transcribe",
// section "CPU weight offload").
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kCThreads = 256;

// grid (T, G): workgroup (t, gy) sums column groups of four gy * kCThreads +
// tid, stepping by G * kCThreads (G spreads a token over several workgroups
// for small batches).  The K row loads of a group are issued together (a
// dropped slot reads row 0 and is not added), then added in slot order.
// y_mode: kYBF16 writes bf16, kYF32 fp32, kYF32Add adds the sum to the fp32
// values y already holds (y_t + sum, one fp32 addition).
template <int K>
__global__ __launch_bounds__(kCThreads) void combine_kernel(const float* __restrict__ rows,
                                                            const int32_t* __restrict__ inv,
                                                            int H, void* y, int y_mode) {
  const int t = blockIdx.x;
  int src[K];
#pragma unroll
  for (int j = 0; j < K; ++j) src[j] = inv[static_cast<size_t>(t) * K + j];
  const int h4 = H / 4;
  for (int c = blockIdx.y * kCThreads + threadIdx.x; c < h4; c += gridDim.y * kCThreads) {
    f32x4 v[K];
#pragma unroll
    for (int j = 0; j < K; ++j)
      v[j] = reinterpret_cast<const f32x4*>(rows + static_cast<size_t>(src[j] < 0 ? 0 : src[j]) * H)[c];
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (src[j] >= 0) s += v[j];
    if (y_mode != kYBF16) {
      f32x4* yo = reinterpret_cast<f32x4*>(static_cast<float*>(y) + static_cast<size_t>(t) * H) + c;
      if (y_mode == kYF32Add) s = *yo + s;
      *yo = s;
    } else {
      const uint32_t lo = f32_to_bf16(s[0]) | (static_cast<uint32_t>(f32_to_bf16(s[1])) << 16);
      const uint32_t hi = f32_to_bf16(s[2]) | (static_cast<uint32_t>(f32_to_bf16(s[3])) << 16);
      reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + static_cast<size_t>(t) * H)[c] =
          make_uint2(lo, hi);
    }
  }
}

// out = bf16(x / sqrt(mean(x^2) + 1e-6)), evaluated in double and rounded once
// Pre-norm of one token per workgroup.  Thread i handles the 8-element
// chunks i, i + kCThreads, ... of the row (16-byte loads and stores); its
// float64 sum of squares runs over its chunks in order, then across the
// wave and the waves.  residual_prenorm_kernel uses the same order, so the
// two give identical results.
__device__ __forceinline__ double block_sum_f64(double ss, double* part) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kCThreads / 64; ++w) tot += part[w];
  return tot;
}

__device__ __forceinline__ double sum_sq8(const u32x4 v) {
  double ss = 0.0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const double lo = bf16_to_f32(v[w] & 0xffffu), hi = bf16_to_f32(v[w] >> 16);
    ss += lo * lo;
    ss += hi * hi;
  }
  return ss;
}

// out chunk = bf16(x / d) for the 8 values of v
__device__ __forceinline__ u32x4 scale8(const u32x4 v, double d) {
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = f64_to_bf16(static_cast<double>(bf16_to_f32(v[w] & 0xffffu)) / d);
    const uint32_t hi = f64_to_bf16(static_cast<double>(bf16_to_f32(v[w] >> 16)) / d);
    o[w] = lo | (hi << 16);
  }
  return o;
}

__global__ __launch_bounds__(kCThreads) void prenorm_kernel(const uint16_t* __restrict__ x, int H,
                                                            uint16_t* __restrict__ out) {
  __shared__ double part[kCThreads / 64];
  const int h8 = H / 8;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(blockIdx.x) * H);
  double ss = 0.0;
  for (int c = threadIdx.x; c < h8; c += kCThreads) ss += sum_sq8(xr[c]);
  const double d = sqrt(block_sum_f64(ss, part) / static_cast<double>(H) + 1e-6);
  u32x4* o = reinterpret_cast<u32x4*>(out + static_cast<size_t>(blockIdx.x) * H);
  for (int c = threadIdx.x; c < h8; c += kCThreads) o[c] = scale8(xr[c], d);
}

__global__ __launch_bounds__(kCThreads) void residual_kernel(uint16_t* __restrict__ x,
                                                             const float* __restrict__ y,
                                                             size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * kCThreads + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * kCThreads)
    x[i] = f64_to_bf16(static_cast<double>(bf16_to_f32(x[i])) + static_cast<double>(y[i]));
}

// Between stacked layers: x = bf16(x + y), then out = bf16(x / sqrt(mean(x^2) +
// 1e-6)) of the new x, one row per workgroup.  Same per-element arithmetic and
// the same reduction order as residual_kernel followed by prenorm_kernel.
__global__ __launch_bounds__(kCThreads) void residual_prenorm_kernel(uint16_t* __restrict__ x,
                                                                     const float* __restrict__ y,
                                                                     int H,
                                                                     uint16_t* __restrict__ out) {
  __shared__ double part[kCThreads / 64];
  const int h8 = H / 8;
  u32x4* xr = reinterpret_cast<u32x4*>(x + static_cast<size_t>(blockIdx.x) * H);
  const f32x4* yr = reinterpret_cast<const f32x4*>(y + static_cast<size_t>(blockIdx.x) * H);
  double ss = 0.0;
  for (int c = threadIdx.x; c < h8; c += kCThreads) {
    const u32x4 v = xr[c];
    const f32x4 y0 = yr[2 * c], y1 = yr[2 * c + 1];
    u32x4 n;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float ylo = w < 2 ? y0[2 * w] : y1[2 * w - 4];
      const float yhi = w < 2 ? y0[2 * w + 1] : y1[2 * w - 3];
      const uint32_t lo =
          f64_to_bf16(static_cast<double>(bf16_to_f32(v[w] & 0xffffu)) + static_cast<double>(ylo));
      const uint32_t hi =
          f64_to_bf16(static_cast<double>(bf16_to_f32(v[w] >> 16)) + static_cast<double>(yhi));
      n[w] = lo | (hi << 16);
    }
    xr[c] = n;
    ss += sum_sq8(n);
  }
  const double d = sqrt(block_sum_f64(ss, part) / static_cast<double>(H) + 1e-6);
  u32x4* o = reinterpret_cast<u32x4*>(out + static_cast<size_t>(blockIdx.x) * H);
  for (int c = threadIdx.x; c < h8; c += kCThreads) o[c] = scale8(xr[c], d);  // written above by this thread
}

}  // namespace

hipError_t launch_combine(const float* rows, const int32_t* inv, int T, int k, int H, void* y,
                          int y_mode, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  // small batches: one column block per workgroup (a single round of loads);
  // large batches: one workgroup per token
  const int g = T < 512 ? (H / 4 + kCThreads - 1) / kCThreads : 1;
  const dim3 grid(T, g);
  switch (k) {
#define MOE_COMBINE_K(KK)                                                                       \
  case KK:                                                                                      \
    hipLaunchKernelGGL(combine_kernel<KK>, grid, dim3(kCThreads), 0, stream, rows, inv, H, y, \
                       y_mode);                                                                 \
    break;
    MOE_COMBINE_K(1) MOE_COMBINE_K(2) MOE_COMBINE_K(3) MOE_COMBINE_K(4)
    MOE_COMBINE_K(5) MOE_COMBINE_K(6) MOE_COMBINE_K(7) MOE_COMBINE_K(8)
#undef MOE_COMBINE_K
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prenorm(const uint16_t* x, int T, int H, uint16_t* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(prenorm_kernel, dim3(T), dim3(kCThreads), 0, stream, x, H, out);
  return hipGetLastError();
}

hipError_t launch_residual(uint16_t* x, const float* y, int T, int H, hipStream_t stream) {
  const size_t n = static_cast<size_t>(T) * H;
  if (n == 0) return hipSuccess;
  size_t g = (n + kCThreads - 1) / kCThreads;
  if (g > 8192) g = 8192;
  hipLaunchKernelGGL(residual_kernel, dim3(static_cast<unsigned>(g)), dim3(kCThreads), 0, stream,
                     x, y, n);
  return hipGetLastError();
}

hipError_t launch_residual_prenorm(uint16_t* x, const float* y, int T, int H, uint16_t* out,
                                   hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(residual_prenorm_kernel, dim3(T), dim3(kCThreads), 0, stream, x, y, H, out);
  return hipGetLastError();
}

}  // namespace moe
