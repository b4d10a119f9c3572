// Per-tensor quantisers for the FP8 (scalar-scale E4M3, W8A8) and 4-bit
// (NVFP4, W4A4) expert formats (bloomery issue #967, section 2 "Checkpoint
// facts"; section 6 keeps each release's W8A8/W4A4 activation rules).
//
// Recipes, each step an IEEE float32 operation:
//   FP8   s = amax / 448,  inv = 448 / amax,  code = E4M3(v * inv)
//   NVFP4 S = amax / 2688 (= 6 * 448),  per 16-element block along K:
//         sb = E4M3(amax_b / (6 * S)); sb == 0 -> zero block;
//         r = 1 / (dec(sb) * S),  code = E2M1(v * r)
//   amax == 0 -> zero codes and a zero scale.
// The same kernels pack expert weights (one scale per expert projection) and
// quantise activations inside the forward pass (one scale per tensor).
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kQThreads = 256;

__global__ __launch_bounds__(kQThreads) void zero_u32_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * kQThreads + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// amax over rows [0, n_rows) of a bf16 [rows, cols] tensor into kAmaxSlots
// slots; 8 elements per thread step
__global__ __launch_bounds__(kQThreads) void amax_bf16_kernel(const uint16_t* __restrict__ x,
                                                              const int32_t* n_rows_dev, int rows,
                                                              int cols, uint32_t* amax) {
  const int nr = n_rows_dev ? min(*n_rows_dev, rows) : rows;
  const size_t n8 = static_cast<size_t>(nr) * cols / 8;
  float m = 0.f;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kQThreads + threadIdx.x; i < n8;
       i += static_cast<size_t>(gridDim.x) * kQThreads) {
    const u32x4 v = reinterpret_cast<const u32x4*>(x)[i];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      m = fmaxf(m, fabsf(bf16_to_f32(v[w] & 0xffffu)));
      m = fmaxf(m, fabsf(bf16_to_f32(v[w] >> 16)));
    }
  }
  block_amax_to_slots(m, amax);
}

// FP8: 8 elements (one 16-byte load) per thread step, so a wave moves 1 KB
// of contiguous input per load.  mode 0 writes dec(code) as bf16 (exact)
// into deq; mode 1 writes the codes.
// One workgroup of kFusedThreads quantises inputs of at most kFusedMaxChunks
// 8-element chunks (16 tokens of 2688) and takes the tensor amax itself: one
// launch instead of the amax kernel and the quantiser (FP8, 4 tokens: step
// 66.7 -> 64.5 us).  At 64 tokens one workgroup was slower than the two
// launches (FP8 step 193 -> 199 us).  The amax is a max, so the codes are the
// same either way.
constexpr int kFusedThreads = 1024;
constexpr size_t kFusedMaxChunks = 16 * 2688 / 8;

// max |x| over n8 chunks of 8 bf16 values, by the whole (single) workgroup
__device__ float block_amax_bf16(const uint16_t* __restrict__ x, size_t n8) {
  __shared__ float part[kFusedThreads / 64];
  float m = 0.f;
  for (size_t i = threadIdx.x; i < n8; i += blockDim.x) {
    const u32x4 v = reinterpret_cast<const u32x4*>(x)[i];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      m = fmaxf(m, fabsf(bf16_to_f32(v[w] & 0xffffu)));
      m = fmaxf(m, fabsf(bf16_to_f32(v[w] >> 16)));
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = 0.f;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) r = fmaxf(r, part[w]);
  return r;
}

template <bool FUSED>
__global__ __launch_bounds__(FUSED ? kFusedThreads : kQThreads) void quant_fp8_kernel(
    const uint16_t* __restrict__ x, const int32_t* n_rows_dev, int rows, int cols,
    const uint32_t* amax_p, int mode, uint16_t* __restrict__ deq, uint8_t* __restrict__ codes,
    float* scale) {
  const int nr = n_rows_dev ? min(*n_rows_dev, rows) : rows;
  const size_t n8 = static_cast<size_t>(nr) * cols / 8;
  float amax;
  if constexpr (FUSED) amax = block_amax_bf16(x, n8);
  else amax = read_amax_slots(amax_p);
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = amax > 0.f ? __fdiv_rn(amax, 448.f) : 0.f;
  // amax == 0: inv = 0, every product is +-0 and every code 0
  const float inv = amax > 0.f ? __fdiv_rn(448.f, amax) : 0.f;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n8;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const u32x4 v = reinterpret_cast<const u32x4*>(x)[i];
    uint32_t c[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t a = v[2 * h], b = v[2 * h + 1];
      c[h] = e4m3_encode4(__uint_as_float(a << 16) * inv, __uint_as_float(a & 0xffff0000u) * inv,
                          __uint_as_float(b << 16) * inv, __uint_as_float(b & 0xffff0000u) * inv);
    }
    if (mode == 0) {
      // every E4M3 value is a bf16 value: the hardware expansion is exact
      const bf16x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, false);
      const bf16x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, true);
      const bf16x2 d2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, false);
      const bf16x2 d3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, true);
      reinterpret_cast<u32x4*>(deq)[i] =
          u32x4{__builtin_bit_cast(uint32_t, d0), __builtin_bit_cast(uint32_t, d1),
                __builtin_bit_cast(uint32_t, d2), __builtin_bit_cast(uint32_t, d3)};
    } else {
      reinterpret_cast<uint2*>(codes)[i] = make_uint2(c[0], c[1]);
    }
  }
}

// NVFP4: 8 elements per thread step; the two halves of a 16-element block sit
// on neighbouring lanes (i even and i + 1), which exchange their amax with
// one DPP move.  n8 is even (cols is a multiple of 16) and the grid stride is
// a multiple of 64, so both halves of a block are in the same wave and the
// same loop iteration.  mode 0 writes the fp16 values dec(q) * dec(sb) into
// deq, which may alias x (at most 6 significant bits and inside [2^-10,
// 2688]: exact in fp16, the operand type of the NVFP4 GEMM); mode 1 writes
// packed codes and block scale codes.
template <bool FUSED>
__global__ __launch_bounds__(FUSED ? kFusedThreads : kQThreads) void quant_nvfp4_kernel(
    const uint16_t* x, const int32_t* n_rows_dev, int rows, int cols, const uint32_t* amax_p,
    int mode, uint16_t* deq, uint8_t* __restrict__ codes, uint8_t* __restrict__ bs,
    float* scale) {
  const int nr = n_rows_dev ? min(*n_rows_dev, rows) : rows;
  const size_t n8 = static_cast<size_t>(nr) * cols / 8;
  float amax;
  if constexpr (FUSED) amax = block_amax_bf16(x, n8);  // read in full before deq may overwrite x
  else amax = read_amax_slots(amax_p);
  const float S = amax > 0.f ? __fdiv_rn(amax, 2688.f) : 0.f;
  if (blockIdx.x == 0 && threadIdx.x == 0 && scale) *scale = S;
  const float sixS = 6.f * S;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n8;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const u32x4 u = reinterpret_cast<const u32x4*>(x)[i];
    float v[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      v[2 * w] = __uint_as_float(u[w] << 16);
      v[2 * w + 1] = __uint_as_float(u[w] & 0xffff0000u);
    }
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    // quad_perm [1, 0, 3, 2]: the value of the neighbouring lane
    const float mo = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, m), 0xb1, 0xf, 0xf, false));
    const float amax_b = fmaxf(m, mo);
    uint32_t sb = 0u;
    float sbf = 0.f;
    if (S > 0.f) {
      sb = e4m3_encode(__fdiv_rn(amax_b, sixS));
      sbf = e4m3_decode(sb);
    }
    // sb == 0: r = 0, every product is +-0 and every code 0
    const float r = sbf > 0.f ? __fdiv_rn(1.f, sbf * S) : 0.f;
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = v[j] * r;
    const uint32_t q = e2m1_encode8(t);
    if (mode == 0) {
      const _Float16 sh = static_cast<_Float16>(sbf);  // E4M3 values are fp16 values
      const f16x2 s2 = {sh, sh};
      const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * s2;
      const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * s2;
      const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * s2;
      const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * s2;
      reinterpret_cast<u32x4*>(deq)[i] =
          u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
    } else {
      reinterpret_cast<uint32_t*>(codes)[i] = q;
      if (!(i & 1)) bs[i >> 1] = static_cast<uint8_t>(sb);
    }
  }
}

// ---- expert weights: per-expert amax into s (as bits), codes, then scales
__global__ __launch_bounds__(kQThreads) void weight_amax_kernel(const uint16_t* __restrict__ w,
                                                                size_t per_expert,
                                                                uint32_t* amax) {
  const int e = blockIdx.y;
  const uint16_t* base = w + static_cast<size_t>(e) * per_expert;
  const size_t n8 = per_expert / 8;
  float m = 0.f;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kQThreads + threadIdx.x; i < n8;
       i += static_cast<size_t>(gridDim.x) * kQThreads) {
    const u32x4 v = reinterpret_cast<const u32x4*>(base)[i];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m = fmaxf(m, fabsf(bf16_to_f32(v[q] & 0xffffu)));
      m = fmaxf(m, fabsf(bf16_to_f32(v[q] >> 16)));
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) atomic_max_nonneg(amax + e, m);
}

__global__ __launch_bounds__(kQThreads) void weight_codes_kernel(
    int fmt, const uint16_t* __restrict__ w, int N, int K, const uint32_t* amax,
    uint8_t* __restrict__ q, uint8_t* __restrict__ bs, int fp8_panels) {
  const size_t per_expert = static_cast<size_t>(N) * K;
  const int e = blockIdx.y;
  const float a = __uint_as_float(amax[e]);
  const uint16_t* base = w + static_cast<size_t>(e) * per_expert;
  const size_t n16 = per_expert / 16;
  if (fmt == kFP8) {
    const float inv = a > 0.f ? __fdiv_rn(448.f, a) : 0.f;
    uint8_t* qe = q + static_cast<size_t>(e) * per_expert;
    for (size_t i = static_cast<size_t>(blockIdx.x) * kQThreads + threadIdx.x; i < n16;
         i += static_cast<size_t>(gridDim.x) * kQThreads) {
      const u32x4 v0 = reinterpret_cast<const u32x4*>(base)[2 * i];
      const u32x4 v1 = reinterpret_cast<const u32x4*>(base)[2 * i + 1];
      uint32_t out[4];
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const uint32_t x0 = ww < 2 ? v0[2 * ww] : v1[2 * (ww - 2)];
        const uint32_t x1 = ww < 2 ? v0[2 * ww + 1] : v1[2 * (ww - 2) + 1];
        uint32_t c[4] = {0u, 0u, 0u, 0u};
        if (a > 0.f) {
          c[0] = e4m3_encode(bf16_to_f32(x0 & 0xffffu) * inv);
          c[1] = e4m3_encode(bf16_to_f32(x0 >> 16) * inv);
          c[2] = e4m3_encode(bf16_to_f32(x1 & 0xffffu) * inv);
          c[3] = e4m3_encode(bf16_to_f32(x1 >> 16) * inv);
        }
        out[ww] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      }
      // chunk i = 16 codes of row n; row-major, or in the panel layout (rows
      // of a panel contiguous per K step of up to 128 codes)
      size_t at = i * 16;
      if (fp8_panels) {
        const size_t n = i / static_cast<size_t>(K / 16);
        const int b = static_cast<int>(i - n * static_cast<size_t>(K / 16));
        const int p = static_cast<int>(n / kNvPanel), pr = static_cast<int>(n % kNvPanel);
        const int rows_p = nv_panel_rows(N, p);
        const int st = b / (kFp8StepK / 16), bq = b % (kFp8StepK / 16);
        const int step_bytes = min(kFp8StepK, K - st * kFp8StepK);
        at = static_cast<size_t>(p) * kNvPanel * K + static_cast<size_t>(st) * rows_p * kFp8StepK +
             static_cast<size_t>(pr) * step_bytes + bq * 16;
      }
      *reinterpret_cast<u32x4*>(qe + at) = u32x4{out[0], out[1], out[2], out[3]};
    }
  } else {
    const float S = a > 0.f ? __fdiv_rn(a, 2688.f) : 0.f;
    const float sixS = 6.f * S;
    uint8_t* qe = q + static_cast<size_t>(e) * (per_expert / 2);
    uint8_t* be = bs + static_cast<size_t>(e) * (per_expert / 16);
    for (size_t i = static_cast<size_t>(blockIdx.x) * kQThreads + threadIdx.x; i < n16;
         i += static_cast<size_t>(gridDim.x) * kQThreads) {
      const u32x4 v0 = reinterpret_cast<const u32x4*>(base)[2 * i];
      const u32x4 v1 = reinterpret_cast<const u32x4*>(base)[2 * i + 1];
      float v[16];
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        v[2 * ww] = bf16_to_f32(v0[ww] & 0xffffu);
        v[2 * ww + 1] = bf16_to_f32(v0[ww] >> 16);
        v[8 + 2 * ww] = bf16_to_f32(v1[ww] & 0xffffu);
        v[8 + 2 * ww + 1] = bf16_to_f32(v1[ww] >> 16);
      }
      float amax_b = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) amax_b = fmaxf(amax_b, fabsf(v[j]));
      uint32_t sb = 0u;
      float sbf = 0.f;
      if (S > 0.f) {
        sb = e4m3_encode(__fdiv_rn(amax_b, sixS));
        sbf = e4m3_decode(sb);
      }
      uint32_t p0 = 0u, p1 = 0u;
      if (sbf > 0.f) {
        const float r = __fdiv_rn(1.f, sbf * S);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p0 |= (e2m1_encode(v[2 * j] * r) | (e2m1_encode(v[2 * j + 1] * r) << 4)) << (8 * j);
          p1 |= (e2m1_encode(v[8 + 2 * j] * r) | (e2m1_encode(v[8 + 2 * j + 1] * r) << 4))
                << (8 * j);
        }
      }
      // block i = row n, block b of the row; stored in the panel layout (rows
      // of a panel contiguous per 64-element K step: 32 code bytes, 4 scales)
      const size_t n = i / static_cast<size_t>(K / 16);
      const int b = static_cast<int>(i - n * static_cast<size_t>(K / 16));
      const int p = static_cast<int>(n / kNvPanel), pr = static_cast<int>(n % kNvPanel);
      const int rows_p = nv_panel_rows(N, p);
      const int st = b / (kNvStepK / 16), bq = b % (kNvStepK / 16);
      const size_t pn0 = static_cast<size_t>(p) * kNvPanel;
      const size_t code_at = pn0 * (K / 2) + static_cast<size_t>(st) * rows_p * (kNvStepK / 2) +
                             static_cast<size_t>(pr) * (kNvStepK / 2) + bq * 8;
      const size_t scale_at = pn0 * (K / 16) + static_cast<size_t>(st) * rows_p * (kNvStepK / 16) +
                              static_cast<size_t>(pr) * (kNvStepK / 16) + bq;
      *reinterpret_cast<uint2*>(qe + code_at) = make_uint2(p0, p1);
      be[scale_at] = static_cast<uint8_t>(sb);
    }
  }
}

__global__ void weight_scales_kernel(int fmt, int E, float* s) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const float a = __uint_as_float(reinterpret_cast<uint32_t*>(s)[e]);
  s[e] = a > 0.f ? __fdiv_rn(a, fmt == kFP8 ? 448.f : 2688.f) : 0.f;
}

int grid_for(size_t work, int cap) {
  size_t b = (work + kQThreads - 1) / kQThreads;
  if (b < 1) b = 1;
  return static_cast<int>(b < static_cast<size_t>(cap) ? b : cap);
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((n + kQThreads - 1) / kQThreads), dim3(kQThreads), 0,
                     stream, p, n);
  return hipGetLastError();
}

hipError_t launch_amax_bf16(const uint16_t* x, const int32_t* n_rows_dev, int rows, int cols,
                            uint32_t* amax, hipStream_t stream) {
  const int grid = grid_for(static_cast<size_t>(rows) * cols / 8, 1024);
  hipLaunchKernelGGL(amax_bf16_kernel, dim3(grid), dim3(kQThreads), 0, stream, x, n_rows_dev,
                     rows, cols, amax);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const uint16_t* x, const int32_t* n_rows_dev, int rows, int cols,
                            const uint32_t* amax, int mode, uint16_t* deq, uint8_t* codes,
                            float* scale, hipStream_t stream) {
  const int grid = grid_for(static_cast<size_t>(rows) * cols / 8, 4096);
  hipLaunchKernelGGL(quant_fp8_kernel<false>, dim3(grid), dim3(kQThreads), 0, stream, x, n_rows_dev,
                     rows, cols, amax, mode, deq, codes, scale);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const uint16_t* x, const int32_t* n_rows_dev, int rows, int cols,
                              const uint32_t* amax, int mode, uint16_t* deq, uint8_t* codes,
                              uint8_t* bs, float* scale, hipStream_t stream) {
  const int grid = grid_for(static_cast<size_t>(rows) * cols / 8, 4096);
  hipLaunchKernelGGL(quant_nvfp4_kernel<false>, dim3(grid), dim3(kQThreads), 0, stream, x, n_rows_dev,
                     rows, cols, amax, mode, deq, codes, bs, scale);
  return hipGetLastError();
}

hipError_t launch_quant_tensor(int fmt, const uint16_t* x, int rows, int cols, uint32_t* amax,
                               int mode, uint16_t* deq, uint8_t* codes, uint8_t* bs, float* scale,
                               hipStream_t stream) {
  const size_t n8 = static_cast<size_t>(rows) * cols / 8;
  if (n8 == 0) return hipSuccess;
  if (n8 <= kFusedMaxChunks) {
    if (fmt == kFP8)
      hipLaunchKernelGGL(quant_fp8_kernel<true>, dim3(1), dim3(kFusedThreads), 0, stream, x,
                         nullptr, rows, cols, nullptr, mode, deq, codes, scale);
    else
      hipLaunchKernelGGL(quant_nvfp4_kernel<true>, dim3(1), dim3(kFusedThreads), 0, stream, x,
                         nullptr, rows, cols, nullptr, mode, deq, codes, bs, scale);
    return hipGetLastError();
  }
  hipError_t err = launch_amax_bf16(x, nullptr, rows, cols, amax, stream);
  if (err != hipSuccess) return err;
  if (fmt == kFP8) return launch_quant_fp8(x, nullptr, rows, cols, amax, mode, deq, codes, scale, stream);
  return launch_quant_nvfp4(x, nullptr, rows, cols, amax, mode, deq, codes, bs, scale, stream);
}

hipError_t launch_quant_weights(int fmt, const uint16_t* w, int E, int N, int K, uint8_t* q,
                                uint8_t* bs, float* s, int fp8_panels, hipStream_t stream) {
  const size_t per = static_cast<size_t>(N) * K;
  hipError_t err = launch_zero_u32(reinterpret_cast<uint32_t*>(s), E, stream);
  if (err != hipSuccess) return err;
  const int gx = grid_for(per / 8, 64);
  hipLaunchKernelGGL(weight_amax_kernel, dim3(gx, E), dim3(kQThreads), 0, stream, w, per,
                     reinterpret_cast<uint32_t*>(s));
  const int gq = grid_for(per / 16, 64);
  hipLaunchKernelGGL(weight_codes_kernel, dim3(gq, E), dim3(kQThreads), 0, stream, fmt, w, N, K,
                     reinterpret_cast<const uint32_t*>(s), q, bs, fp8_panels);
  hipLaunchKernelGGL(weight_scales_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, fmt, E,
                     s);
  return hipGetLastError();
}

}  // namespace moe
