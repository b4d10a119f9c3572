/*
 * moe.h -- C ABI of libmoe.so: the routed mixture-of-experts layer of the
 * Nemotron 3.5 Transcribe hybrid decoder on AMD Instinct MI355X (gfx950).
 *
 * The layer (bloomery issue #967 "model: Nemotron 3.5 Transcribe from
 * safetensors on x86 cards and DGX Spark", section 2 "Checkpoint facts";
 * section 3 "Existing owners and gaps"):
 *   width H = 2688, E = 128 experts, top-k = 6 routing, ungated ReLU^2 experts
 *   of width F = 1856 (an up part H->F and a down part F->H, no gate matrix);
 *   expert weights in BF16, FP8 (scalar-scale E4M3, W8A8) or 4-bit NVFP4
 *   (W4A4).
 * Routing is a separate formula from expert execution (audio.cpp port notes
 * "NVIDIA Nemotron 3.5 Transcribe", section "CPU weight offload"), hence two
 * calls: moe_route and moe_forward.
 *
 * Conventions for every call:
 *   - Pointers marked [dev] are device pointers (hipMalloc or torch CUDA
 *     tensors); [host] are host pointers read during the call only (except
 *     a cache's host bank, which its uploads read from `stream` later: keep
 *     it unchanged while they may be in flight).
 *   - All device work is enqueued asynchronously on `stream` (a hipStream_t;
 *     NULL = the null stream).  No call synchronises with the host, except
 *     moe_cache_init and moe_forward_cached, which wait for `stream`.
 *   - Row-major, contiguous layouts, except the packed NVFP4 expert bank
 *     (128-row panels, see moe_experts); bf16 is passed as raw 16-bit words.
 *   - Alignment: token rows (x), outputs (y), router and expert weight codes
 *     are read and written in 16-byte vectors, so those pointers must be
 *     16-byte aligned; ids, gates, biases, scales and block scales 4-byte
 *     aligned; FP8 activation codes 8-byte aligned.  A misaligned pointer
 *     is MOE_EINVAL (hipMalloc and torch allocations are 256-byte aligned).
 *   - The caller owns every buffer.  The library allocates no device memory;
 *     scratch comes from the caller's workspace (moe_workspace_size).
 *   - Arguments are validated on the host before any launch.  On error the
 *     call returns a non-zero moe_status and enqueues nothing (one
 *     exception: moe_forward_cached reports a batch that selects more
 *     experts than the cache holds after its permutation).  T == 0 is a
 *     valid no-op.  A failed launch returns MOE_EHIP.
 *   - Calls are reentrant; calls that share a workspace must be ordered on
 *     one stream.  Non-finite inputs give undefined (but memory-safe)
 *     results.  Expert ids outside [0, E) are dropped by moe_forward (their
 *     slot contributes nothing).
 *   - Supported shapes: 64 <= H, 64 <= F with H % 64 == F % 64 == 0,
 *     16 <= E <= 256 with E % 16 == 0, 1 <= top_k <= min(8, E),
 *     0 <= T <= 1 << 20.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 7

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,       /* bad argument: null pointer, bad size or enum   */
  MOE_EUNSUPPORTED = 2, /* valid request outside the supported shapes    */
  MOE_EWORKSPACE = 3,   /* workspace missing or smaller than required    */
  MOE_EHIP = 4          /* a HIP launch or runtime call failed           */
} moe_status;

/* Expert weight formats (bloomery issue #967, section 2 "Checkpoint facts":
 * BF16, FP8 scalar-scale E4M3 W8A8, NVFP4 W4A4 experts). */
typedef enum {
  MOE_WFMT_BF16 = 0,
  MOE_WFMT_FP8 = 1,   /* E4M3 codes, one fp32 scale per expert projection;
                         activations quantised per tensor to E4M3          */
  MOE_WFMT_NVFP4 = 2  /* E2M1 codes in 16-element blocks along K, one E4M3
                         scale per block, one fp32 scale per expert
                         projection; activations quantised the same way    */
} moe_wfmt;

typedef enum { MOE_Y_BF16 = 0, MOE_Y_F32 = 1 } moe_ydtype;

/* [host] layer shape: hidden H, expert width F, experts E, experts per token k */
typedef struct {
  int32_t hidden, ffn, n_experts, top_k;
} moe_dims;

/* [host] struct of [dev] router tensors: w_packed bf16 [3, E, H] written by
 * moe_router_pack from the fp32 router matrix; bias fp32 [E] or NULL */
typedef struct {
  const void* w_packed;
  const float* bias;
} moe_router;

/* [host] struct of [dev] expert bank pointers.
 *   BF16 : up  bf16 [E, F, H],  down bf16 [E, H, F]
 *   FP8  : up  u8 E4M3 [E, F, H] row-major; down u8 H*F bytes per expert
 *          in 128-row panels (below); up_s/down_s fp32 [E]
 *          (weight = dec(code) * s).  Down panels: the H x F matrix is cut
 *          into panels of rows_p = min(128, H - 128 p) rows, each stored
 *          K-step-major in steps of 128 codes (the last step 64 codes when
 *          F % 128 == 64): code j of row n, step s lies at
 *            128 p * F + s * rows_p * 128 + (n - 128 p) * sb + j,
 *          sb = min(128, F - 128 s), p = n / 128, from the expert's base, so
 *          every step of a row is one aligned 128-byte line (F = 1856 rows
 *          are 14.5 lines; row-major, half of them would straddle lines).
 *   NVFP4: up  u8 F*H/2 bytes per expert, down u8 H*F/2 (two E2M1 codes per
 *          byte, element 2i in the low nibble); up_bs u8 E4M3 F*H/16 bytes
 *          per expert, down_bs H*F/16 (one per 16-element block along K);
 *          up_s/down_s fp32 [E]  (weight = dec(code) * dec(block scale) * s).
 *          Panel layout: a projection's N x K matrix is cut into panels of
 *          128 rows (the last may be shorter, rows_p = min(128, N - 128 p))
 *          and each panel is stored K-step-major in steps of 64 elements.
 *          Code byte j (0..31) of row n, step s lies at
 *            128 p * K/2 + s * rows_p * 32 + (n - 128 p) * 32 + j,
 *          block scale j (0..3) of row n, step s at
 *            128 p * K/16 + s * rows_p * 4 + (n - 128 p) * 4 + j,
 *          p = n / 128, from the expert's base.  moe_quantize_experts
 *          writes this layout; a GEMM tile then reads one contiguous block
 *          per K step.
 * Unused pointers may be NULL. */
typedef struct {
  int32_t fmt; /* moe_wfmt */
  const void* up;
  const void* down;
  const uint8_t* up_bs;
  const uint8_t* down_bs;
  const float* up_s;
  const float* down_s;
} moe_experts;

/* MOE_ABI_VERSION of the built library. */
int32_t moe_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* moe_status_str(int32_t status);

/* Bytes of workspace moe_forward needs for up to `max_tokens` tokens with
 * weight format `fmt`; 0 for invalid arguments.  The workspace must be
 * 256-byte aligned (hipMalloc and torch allocations are). */
size_t moe_workspace_size(const moe_dims* dims, int32_t fmt, int32_t max_tokens);

/* Pack the fp32 router matrix w [dev] [E, H] for moe_route: w_packed [dev]
 * bf16 [3, E, H] = (hi, mid, lo) with w == hi + mid + lo exactly (hi and mid
 * are truncations, lo holds the remaining <= 8 significant bits), so the
 * router's products with bf16 tokens are exact on bf16 MFMA.  Run once per
 * router matrix. */
int32_t moe_router_pack(const moe_dims* dims, const float* w, void* w_packed,
                        void* stream);

/* Bytes of workspace moe_route needs for up to `max_tokens` tokens (partial
 * logits); 0 for invalid arguments. */
size_t moe_route_workspace_size(const moe_dims* dims, int32_t max_tokens);

/* Router (bloomery issue #967, section 2: top-6 routing over 128 experts;
 * audio.cpp notes, section "CPU weight offload": routing weights are their own
 * formula).  For each token t:
 *   l_t = fp32(x_t) . W_r^T + b                (fp32 accumulation)
 *   ids[t, 0..k) = the k largest l_t,e, ordered by (logit desc, index asc)
 *   gates[t, j]  = exp(l_t,ids[j]) / sum_j' exp(l_t,ids[j'])
 * x [dev] bf16 [T, H]; ids [dev] int32 [T, k] out; gates [dev] fp32 [T, k] out;
 * ws [dev] workspace of ws_bytes >= moe_route_workspace_size(dims, T),
 * 256-byte aligned. */
int32_t moe_route(const moe_dims* dims, int32_t T, const void* x,
                  const moe_router* router, int32_t* ids, float* gates,
                  void* ws, size_t ws_bytes, void* stream);

/* Expert part of the layer (bloomery issue #967, sections 2-3: ungated ReLU^2
 * experts 2688 -> 1856 -> 2688; audio.cpp notes, "CPU weight offload":
 * grouped expert matrix multiplication).  For each token t:
 *   y_t = sum_{j<k} gates[t,j] * W_down,e . a~,   a = bf16(relu(W_up,e . x~_t)^2)
 * with e = ids[t, j], x~ / a~ the activations as the weight format quantises
 * them (identity for BF16; per-tensor E4M3 for FP8; NVFP4 blocks for 4-bit),
 * fp32 accumulation, slots summed in order j = 0..k-1.
 *   x     [dev] bf16 [T, H]        ids [dev] int32 [T, k]    gates [dev] fp32 [T, k]
 *   y     [dev] [T, H], bf16 (MOE_Y_BF16) or fp32 (MOE_Y_F32), written in full
 *   ws    [dev] workspace of ws_bytes >= moe_workspace_size(dims, fmt, T)
 * After the call the workspace holds the stage results described by
 * moe_workspace_layout until the next call that uses it. */
int32_t moe_forward(const moe_dims* dims, int32_t T, const void* x,
                    const int32_t* ids, const float* gates,
                    const moe_experts* experts, void* y, int32_t y_dtype,
                    void* ws, size_t ws_bytes, void* stream);

/* moe_forward with stage timing.  `events` [host] holds n_events >= 7
 * hipEvent_t handles created by the caller (with timing enabled);
 * events[i] is recorded on `stream` before stage i and events[6] after the
 * last one.  Stages: 0 permutation (histogram, prefix sum, scatter), 1 token
 * quantisation (FP8/NVFP4), 2 up projection + ReLU^2, 3 intermediate
 * quantisation (FP8/NVFP4), 4 down projection, 5 combine.
 * With n_events >= 11, events[7], events[8] take the start and end of the up
 * projection kernel itself and events[9], events[10] those of the down
 * projection kernel (stamped from the kernels' dispatch packets through
 * hipExtLaunchKernel, so they exclude the marker packets around a stage; a
 * launch with no tiles records both back to back).  Results are identical
 * to moe_forward.  With T = 0 nothing is enqueued and no event is recorded. */
#define MOE_N_STAGES 6
int32_t moe_forward_timed(const moe_dims* dims, int32_t T, const void* x,
                          const int32_t* ids, const float* gates,
                          const moe_experts* experts, void* y, int32_t y_dtype,
                          void* ws, size_t ws_bytes, void* stream,
                          void* const* events, int32_t n_events);

/* ---- shared expert
 * The pages' decoder keeps shared experts on the card beside the routed ones
 * (bloomery issue #967, section 4 "Placement on card, host RAM and NVMe");
 * they give no width for them.  A shared expert is one ungated ReLU^2 FFN
 * that every token takes with weight 1:
 *   y_t (+)= W_down,s . a~_t,   a = bf16(relu(W_up,s . x~_t)^2)
 * with x~ quantised as in moe_forward (per tensor over x) and a~ per tensor
 * over the shared intermediate [T, F_s] on its own (FP8, NVFP4).
 *   dims   [host] {H, F_s, 1, 1}: hidden width, shared-expert width, one
 *          expert, one slot (MOE_EINVAL otherwise); H, F_s multiples of 64
 *   x      [dev] bf16 [T, H]
 *   expert [host] struct of [dev] pointers: a one-expert bank in the layouts
 *          of moe_experts (E = 1; moe_quantize_experts packs it)
 *   y      [dev] [T, H]: written (accumulate = 0; bf16 or fp32), or with
 *          accumulate = 1 the fp32 result is added to the fp32 values y holds
 *          (y_dtype must be MOE_Y_F32): after moe_forward into y this gives
 *          the MoE block, routed + shared
 *   ws     [dev] workspace of ws_bytes >= moe_shared_workspace_size(dims, fmt, T)
 * Errors as moe_forward; T == 0 is a no-op. */
size_t moe_shared_workspace_size(const moe_dims* dims, int32_t fmt, int32_t max_tokens);
int32_t moe_shared_forward(const moe_dims* dims, int32_t T, const void* x,
                           const moe_experts* expert, void* y, int32_t y_dtype,
                           int32_t accumulate, void* ws, size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace: scratch lives in a fixed device array inside the
 * library, MOE_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs
 * on holds until the process ends (8 MiB: up to 64 tokens at the full layer
 * shape in every format).  The call allocates nothing and calls no
 * allocating routine.  Arguments, results and errors are those of
 * moe_forward, plus:
 *   MOE_EWORKSPACE  moe_workspace_size(dims, fmt, T) exceeds the array
 *   MOE_EINVAL      `stream` belongs to a device other than the current one
 * The array is found on the current device (hipGetDevice) the first time the
 * call runs there.  Every call on one GPU shares that GPU's array, which keeps
 * the last call's stage results: calls that may overlap on one GPU (other
 * streams, other threads) race, so order them on one stream. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int32_t moe_forward_noalloc(const moe_dims* dims, int32_t T, const void* x,
                            const int32_t* ids, const float* gates,
                            const moe_experts* experts, void* y, int32_t y_dtype,
                            void* stream);

/* ---- expert residency split
 * The routed expert banks stay in host memory in their stored format; the
 * experts a batch selects are uploaded into a bounded cache of device slots,
 * and experts that keep being selected stay resident.  The cache must cover
 * the experts selected together and cannot exceed the expert count
 * (audio.cpp notes "NVIDIA Nemotron 3.5 Transcribe", section "CPU weight
 * offload").  Here a batch's touched experts must fit the slots; the least
 * recently used resident experts the batch does not touch are replaced.
 * All memory is the caller's:
 *   host      the whole bank in host memory, layouts as moe_experts (fmt, up,
 *             down, up_bs, down_bs; pinned memory lets the uploads run as
 *             asynchronous DMA); its scale pointers are not used
 *   up_s, down_s  [dev] fp32 [E] per-expert scales (FP8/NVFP4), resident
 *   slot_up, slot_down        [dev] n_slots experts of codes, same
 *             per-expert layout and size as the bank
 *   slot_up_bs, slot_down_bs  [dev] NVFP4 block scales of the slots
 *   slot_of   [dev] int32 [E]: the slot of each expert, written by the library
 *   state     [host] moe_cache_state_size bytes of replacement state,
 *             8-byte aligned, kept by the caller between calls
 * Calls that share a cache (its slots, map or state) must not overlap. */
typedef struct {
  int32_t n_slots;
  moe_experts host;
  const float* up_s;
  const float* down_s;
  void* slot_up;
  void* slot_down;
  uint8_t* slot_up_bs;
  uint8_t* slot_down_bs;
  int32_t* slot_of;
} moe_cache;

/* [host] per-call counters of moe_forward_cached */
typedef struct {
  int32_t touched;          /* experts the batch selected              */
  int32_t hits;             /* of them, already resident               */
  int32_t misses;           /* of them, uploaded by this call          */
  int64_t bytes_uploaded;   /* host-to-device bytes of those uploads   */
} moe_cache_stats;

/* Host bytes of replacement state for n_slots slots (top_k <= n_slots <= E);
 * 0 for invalid arguments. */
size_t moe_cache_state_size(const moe_dims* dims, int32_t n_slots);

/* Marks every slot empty (state, and slot_of on `stream`, which the call
 * waits for).  MOE_EINVAL for null pointers, n_slots outside
 * [top_k, n_experts] or a too small state. */
int32_t moe_cache_init(const moe_dims* dims, const moe_cache* cache, void* state,
                       size_t state_bytes, void* stream);

/* moe_forward with the expert weights taken from the cache.  After the
 * permutation it copies the per-expert row counts to the host and waits for
 * the stream (the uploads depend on the routing), uploads the missing
 * experts, updates slot_of and runs the expert GEMMs on the slots; y equals
 * moe_forward's on the same bank bit for bit.  If the batch selects more
 * experts than there are slots it returns MOE_EUNSUPPORTED after the
 * permutation, with nothing uploaded and y not written.  After MOE_EHIP the
 * cache must be set up again with moe_cache_init.  Not capturable in a HIP
 * graph (it waits for the stream).  stats [host] may be NULL. */
int32_t moe_forward_cached(const moe_dims* dims, int32_t T, const void* x,
                           const int32_t* ids, const float* gates, const moe_cache* cache,
                           void* state, void* y, int32_t y_dtype, void* ws, size_t ws_bytes,
                           void* stream, moe_cache_stats* stats);

/* Byte offsets of stage results inside a moe_forward workspace (for tests and
 * tools; -1 where a stage does not exist for the format). */
typedef struct {
  int64_t counts;     /* int32 [E]: rows routed to each expert               */
  int64_t offsets;    /* int32 [E+1]: exclusive prefix sum of counts         */
  int64_t sorted_src; /* int32 [T*k]: flat (t*k + j) index of each sorted row */
  int64_t inv;        /* int32 [T*k]: sorted row of each flat index, -1 = dropped */
  int64_t act;        /* bf16 [T*k, F]: a = bf16(relu(h)^2), sorted row order */
  int64_t out_rows;   /* fp32 [T*k, H]: gate * W_down a~, sorted row order   */
  int64_t x_q;        /* [T, H] dequantised token values without the tensor
                         scale: FP8 bf16 dec(q); NVFP4 fp16 dec(q)*dec(sb)   */
  int64_t act_q;      /* FP8: u8 [T*k, F] codes; NVFP4: fp16 dec(q)*dec(sb)
                         in place over act                                   */
  int64_t scales;     /* fp32 [2]: x scale, act scale                        */
  int64_t total;      /* bytes                                               */
} moe_ws_layout;

int32_t moe_workspace_layout(const moe_dims* dims, int32_t fmt, int32_t T,
                             moe_ws_layout* out /* [host] */);

/* Pack a bf16 expert bank into FP8 or NVFP4 on the device (any expert count
 * 1 <= E <= 256, e.g. a shared expert's one-expert bank; top_k is not used),
 * one fp32 scale per expert projection (recipes: s = f32(amax/448), code = E4M3(f32(w*f32(448/amax)))
 * for FP8; S = f32(amax/2688), block scale sb = E4M3(f32(amax_b/f32(6S))),
 * code = E2M1(f32(w*f32(1/f32(sb*S)))) for NVFP4; amax == 0 -> zero codes and
 * scale).  Layouts as in moe_experts.
 *   up_bf16 [dev] [E, F, H], down_bf16 [dev] [E, H, F]
 *   up_q, down_q [dev] out; up_bs, down_bs [dev] out (NVFP4 only, else NULL);
 *   up_s, down_s [dev] fp32 [E] out. */
int32_t moe_quantize_experts(const moe_dims* dims, int32_t fmt,
                             const void* up_bf16, const void* down_bf16,
                             void* up_q, void* down_q, uint8_t* up_bs,
                             uint8_t* down_bs, float* up_s, float* down_s,
                             void* stream);

/* Per-tensor activation quantiser of moe_forward as a standalone call (same
 * recipes as moe_quantize_experts, amax over the whole [rows, cols] tensor).
 *   x [dev] bf16 [rows, cols]; codes [dev] u8 [rows, cols] (FP8) or
 *   [rows, cols/2] (NVFP4: two codes per byte as in the weights, row-major);
 *   bs [dev] u8 [rows, cols/16] (NVFP4 only, row-major); scale [dev] fp32 [1] out;
 *   ws [dev] >= 256 bytes of scratch. */
int32_t moe_quantize_activation(int32_t fmt, int32_t rows, int32_t cols,
                                const void* x, void* codes, uint8_t* bs,
                                float* scale, void* ws, size_t ws_bytes,
                                void* stream);

/* Stacked-path helpers.  The pages' model normalises around its layers
 * (audio.cpp notes, section "Q4_K, Q3_K and Q2_K expert profiles": routing and
 * normalisation stay unchanged); a weightless RMS pre-norm is used:
 *   moe_prenorm:           out_t = bf16(x_t / sqrt(mean(x_t^2) + 1e-6))
 *   moe_residual_add:      x_t   = bf16(x_t + y_t)
 *   moe_residual_prenorm:  moe_residual_add, then moe_prenorm of the new x
 *                          into out, in one pass (bit-identical to the two
 *                          calls; for the step between stacked layers)
 * x, out [dev] bf16 [T, H] (out must not be x); y [dev] fp32 [T, H];
 * H % 64 == 0; moe_prenorm and moe_residual_prenorm need 16-byte aligned
 * x, y and out (MOE_EINVAL otherwise).  Row sums of squares are
 * accumulated in double. */
int32_t moe_prenorm(int32_t T, int32_t H, const void* x, void* out, void* stream);
int32_t moe_residual_add(int32_t T, int32_t H, void* x, const float* y, void* stream);
int32_t moe_residual_prenorm(int32_t T, int32_t H, void* x, const float* y, void* out,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
