// Internal launchers of libmoe (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum Fmt { kBF16 = 0, kFP8 = 1, kNVFP4 = 2 };
// GEMM operand modes: kFP8 runs the FP8 MFMA on E4M3 codes; kFP8X expands
// E4M3 weight codes to bf16 (exact) in LDS and runs the BF16 MFMA.
constexpr int kFP8X = 3;

constexpr int kChunk = 2048;  // flat (token, slot) entries per permutation chunk

// NVFP4 expert banks: each expert projection [N, K] is cut into panels of
// kNvPanel rows (the last one may be shorter), and each panel is stored
// K-step-major: for step s (64 elements of K) the panel's rows follow one
// another, 32 code bytes each in the code array and 4 block-scale bytes each
// in the scale array.  Panel p starts where row-major row p * kNvPanel would,
// so the arrays keep their row-major sizes.  A GEMM tile of at most kNvPanel
// columns inside one panel then reads one contiguous block per K step.
constexpr int kNvPanel = 128;
constexpr int kNvStepK = 64;
// FP8 down-projection codes use the same 128-row panels, K-step-major in
// steps of kFp8StepK codes (one 128-byte line per row; a last step of 64
// codes when K % 128 == 64).  Rows of F = 1856 codes are not a whole number
// of lines, so in row-major order half the rows would straddle lines.
constexpr int kFp8StepK = 128;

__host__ __device__ __forceinline__ int nv_panel_rows(int N, int p) {
  const int left = N - p * kNvPanel;
  return left < kNvPanel ? left : kNvPanel;
}

struct PermBufs {
  int32_t* chunk_counts;  // [n_chunks, E]
  int32_t* chunk_base;    // [n_chunks, E]
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E + 1]
  int32_t* sorted_src;    // [R]
  int32_t* inv;           // [R]
  float* row_gate;        // [R]
  int bm0;                // rows per tile, list 0 (up projection)
  int32_t* tile_off0;     // [E + 1]: exclusive prefix of ceil(count_e / bm0)
  int bm1;                // rows per tile, list 1 (down projection)
  int32_t* tile_off1;     // [E + 1]
  uint32_t* zero_words;   // cleared by the scan (amax slots)
  int n_zero;
};

// K slices of the router GEMV for T tokens (partial logits [S, T, E] fp32)
int router_k_slices(int T, int H);
hipError_t launch_router_pack(const float* w, int E, int H, uint16_t* packed, hipStream_t stream);
hipError_t launch_router(const uint16_t* x, const uint16_t* w_packed, const float* bias, int T,
                         int H, int E, int k, float* part, int32_t* ids, float* gates,
                         hipStream_t stream);

hipError_t launch_permute(const int32_t* ids, const float* gates, int T, int E, int k,
                          const PermBufs& p, hipStream_t stream);
// One expert taking every token with weight 1 (the shared expert): the
// permutation is the identity, written without ids or gates.
hipError_t launch_permute_identity(int T, const PermBufs& p, hipStream_t stream);

// Grouped GEMM over the tile list.  Up: out = bf16(relu(scale * A_g W^T)^2)
// with A_g the token rows gathered through sorted_src; down:
// out = fp32(gate * scale * A W^T).
struct GemmArgs {
  const int32_t* tile_off;    // [E + 1]: row tiles of experts < e (bm rows each)
  int E;
  int max_tiles;              // upper bound of tile_off[E] (grid sizing)
  const int32_t* offsets;     // [E + 1]
  const int32_t* sorted_src;  // up only: flat index of each sorted row
  int top_k;
  const void* a;              // up: tokens [T, K]; down: activations [R, K]
  const void* b;              // expert weights, [E, N, K] (nvfp4: N*K/2 bytes per expert
                              // in kNvPanel-row panels, K-step-major)
  const uint8_t* b_bs;        // nvfp4 block scales, N*K/16 bytes per expert, same panels
  const float* b_s;           // fp8 / nvfp4 weight scale per expert [E]
  const int32_t* w_slot;      // [E] slot of each expert's weights in b / b_bs, or null:
                              // expert e at index e (resident bank)
  const float* a_s;           // fp8 / nvfp4 activation scale (device scalar)
  int N, K;
  void* out;                  // up: bf16 [R, N]; down: fp32 [R, N]
  const float* row_gate;      // down only: [R]
  uint32_t* amax;             // up with fp8 / nvfp4: amax of the bf16 output
};

struct GemmShape {
  int bm, bn;
};

// Tile shape the forward pass uses for T tokens (rows per tile feeds the
// permutation's tile lists).
GemmShape gemm_shape(int fmt, int stage, int T);

// Optional timing of one GEMM launch: events that receive the kernel's own
// start and end (from its dispatch packet, not markers around it).
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

hipError_t launch_gemm(int fmt, int stage, int T, const GemmArgs& g, hipStream_t stream,
                       const KernelEvents& ev = KernelEvents{});

// activation quantisers
hipError_t launch_amax_bf16(const uint16_t* x, const int32_t* n_rows_dev, int rows, int cols,
                            uint32_t* amax, hipStream_t stream);
// FP8: codes = E4M3(f32(x * f32(448/amax))); writes scale f32(amax/448) to *scale.
// mode 0: dec(code) as bf16 into deq; mode 1: the codes.
hipError_t launch_quant_fp8(const uint16_t* x, const int32_t* n_rows_dev, int rows, int cols,
                            const uint32_t* amax, int mode, uint16_t* deq, uint8_t* codes,
                            float* scale, hipStream_t stream);
// NVFP4: per 16-block codes and E4M3 scale; writes tensor scale to *scale.
// mode 0: dequantised block values dec(q)*dec(sb) as fp16 into deq (may alias x);
// mode 1: packed codes + block scales.
hipError_t launch_quant_nvfp4(const uint16_t* x, const int32_t* n_rows_dev, int rows, int cols,
                              const uint32_t* amax, int mode, uint16_t* deq, uint8_t* codes,
                              uint8_t* bs, float* scale, hipStream_t stream);
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t stream);

// output modes of the combine: bf16 y, fp32 y, fp32 y += the combined rows
enum YMode { kYBF16 = 0, kYF32 = 1, kYF32Add = 2 };
hipError_t launch_combine(const float* rows, const int32_t* inv, int T, int k, int H, void* y,
                          int y_mode, hipStream_t stream);

// Per-tensor quantisation of a whole bf16 tensor [rows, cols] (the tokens,
// or moe_quantize_activation): amax into the zeroed slots `amax`, then codes
// (FP8: mode 0 bf16 dec(code) into deq, mode 1 codes; NVFP4: mode 0 fp16
// values into deq, mode 1 codes and block scales).  Small tensors run in one
// workgroup that takes the amax itself and leaves the slots untouched.
hipError_t launch_quant_tensor(int fmt, const uint16_t* x, int rows, int cols, uint32_t* amax,
                               int mode, uint16_t* deq, uint8_t* codes, uint8_t* bs, float* scale,
                               hipStream_t stream);

// fp8_panels: write FP8 codes in the panel layout (down projection) rather
// than row-major (up projection)
hipError_t launch_quant_weights(int fmt, const uint16_t* w, int E, int N, int K, uint8_t* q,
                                uint8_t* bs, float* s, int fp8_panels, hipStream_t stream);

hipError_t launch_prenorm(const uint16_t* x, int T, int H, uint16_t* out, hipStream_t stream);
hipError_t launch_residual(uint16_t* x, const float* y, int T, int H, hipStream_t stream);
hipError_t launch_residual_prenorm(uint16_t* x, const float* y, int T, int H, uint16_t* out,
                                   hipStream_t stream);

}  // namespace moe
