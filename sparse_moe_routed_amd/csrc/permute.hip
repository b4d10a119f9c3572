// Token permutation: per-expert histogram, exclusive prefix sum with a
// per-expert GEMM tile counts, and a stable scatter of (token, slot) rows into
// expert-contiguous order.
//
// Grouped expert matrix multiplication needs the rows routed to one expert
// next to each other (audio.cpp notes "NVIDIA Nemotron 3.5 Transcribe",
// section "CPU weight offload").  Row order inside an expert is the flat
// index i = t*k + j (token-major), so the result is deterministic and equals
// a stable sort of the flat ids by expert.
//
// The flat ids are cut into chunks of kChunk entries.  perm_count writes
// per-chunk expert counts; perm_scan (one workgroup) turns them into chunk
// bases, expert offsets and per-expert row-tile prefixes for the GEMMs;
// perm_scatter recomputes each entry's stable rank inside its chunk with wave
// ballots.  When all ids fit one chunk (decode batches) perm_single does the
// three steps in one workgroup.  No host sync.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kPermThreads = 256;
constexpr int kRounds = kChunk / kPermThreads;  // entries per thread per chunk

// this thread's entries of one chunk (round r holds flat index chunk * kChunk
// + r * kPermThreads + threadIdx.x), all loads issued together: the expert id
// when it lies in [0, E), else -1 (also past R)
__device__ __forceinline__ void load_chunk(const int32_t* __restrict__ ids, int R, int E,
                                           int chunk, int (&ev)[kRounds]) {
  const int base = chunk * kChunk;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int i = base + r * kPermThreads + threadIdx.x;
    const int e = i < R ? ids[i] : -1;
    ev[r] = (e >= 0 && e < E) ? e : -1;
  }
}

// per-expert counts of one chunk into LDS cnt[] (zeroed by the caller)
__device__ __forceinline__ void count_chunk(const int (&ev)[kRounds], int32_t* cnt) {
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
    if (ev[r] >= 0) atomicAdd(&cnt[ev[r]], 1);
}

__global__ __launch_bounds__(kPermThreads) void perm_count_kernel(
    const int32_t* __restrict__ ids, int R, int E, int32_t* __restrict__ chunk_counts) {
  __shared__ int32_t cnt[256];
  int ev[kRounds];
  load_chunk(ids, R, E, blockIdx.x, ev);
  for (int e = threadIdx.x; e < E; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  count_chunk(ev, cnt);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads)
    chunk_counts[static_cast<size_t>(blockIdx.x) * E + e] = cnt[e];
}

// block-wide exclusive scan of one value per thread (256 threads)
__device__ int block_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int wbase = 0, sum = 0;
  for (int w = 0; w < kPermThreads / 64; ++w) {
    if (w < wave) wbase += tmp[w];
    sum += tmp[w];
  }
  __syncthreads();
  total = sum;
  return wbase + incl - v;
}

// expert offsets and both GEMM tile prefixes from the total count `run` of
// expert e = threadIdx.x (0 when e >= E); zeroes the words the later stages
// accumulate into
__device__ void scan_experts(int run, int E, int32_t* __restrict__ counts,
                             int32_t* __restrict__ offsets, int bm0, int32_t* __restrict__ tile_off0,
                             int bm1, int32_t* __restrict__ tile_off1,
                             uint32_t* __restrict__ zero_words, int n_zero, int* tmp) {
  const int e = threadIdx.x;
  for (int i = threadIdx.x; i < n_zero; i += kPermThreads) zero_words[i] = 0u;
  if (e < E) counts[e] = run;
  int total;
  const int off = block_exclusive_scan(e < E ? run : 0, tmp, total);
  if (e < E) offsets[e] = off;
  if (e == 0) offsets[E] = total;

  // per-expert row-tile prefix: expert e owns ceil(count / bm) tiles of up to bm rows
  for (int list = 0; list < 2; ++list) {
    const int bm = list ? bm1 : bm0;
    int32_t* tile_off = list ? tile_off1 : tile_off0;
    const int nt = e < E ? (run + bm - 1) / bm : 0;
    int nt_total;
    const int tbase = block_exclusive_scan(nt, tmp, nt_total);
    if (e < E) tile_off[e] = tbase;
    if (e == 0) tile_off[E] = nt_total;
  }
}

__global__ __launch_bounds__(kPermThreads) void perm_scan_kernel(
    const int32_t* __restrict__ chunk_counts, int n_chunks, int E,
    int32_t* __restrict__ chunk_base, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int bm0, int32_t* __restrict__ tile_off0, int bm1,
    int32_t* __restrict__ tile_off1, uint32_t* __restrict__ zero_words, int n_zero) {
  __shared__ int tmp[kPermThreads / 64];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < n_chunks; ++c) {
      const size_t at = static_cast<size_t>(c) * E + e;
      chunk_base[at] = run;
      run += chunk_counts[at];
    }
  }
  scan_experts(run, E, counts, offsets, bm0, tile_off0, bm1, tile_off1, zero_words, n_zero, tmp);
}

// stable scatter of one chunk (entries from load_chunk); run[e] (LDS) holds
// the first sorted row of expert e for this chunk and advances past it.
// Rounds wholly past R are skipped (the test is uniform over the workgroup).
__device__ void scatter_chunk(const int (&ev)[kRounds], const float* __restrict__ gates, int R,
                              int E, int chunk, int32_t* run, int32_t (*wcnt)[256],
                              int32_t* __restrict__ sorted_src, int32_t* __restrict__ inv,
                              float* __restrict__ row_gate) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = chunk * kChunk;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  float gv[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int i = base + r * kPermThreads + threadIdx.x;
    gv[r] = ev[r] >= 0 ? gates[i] : 0.f;
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    if (base + r * kPermThreads >= R) break;
    const int i = base + r * kPermThreads + threadIdx.x;
    const int e = ev[r];
    if (i < R && e < 0) inv[i] = -1;
    // lanes of this wave holding the same expert
    uint64_t same = __ballot(e >= 0);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t bit = __ballot(e >= 0 && ((e >> b) & 1));
      same &= ((e >> b) & 1) ? bit : ~bit;
    }
    const int rank = __popcll(same & lt_mask);
    if (e >= 0 && rank == 0) wcnt[wave][e] = __popcll(same);
    __syncthreads();
    if (e >= 0) {
      int pos = run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      sorted_src[pos] = i;
      inv[i] = pos;
      row_gate[pos] = gv[r];
    }
    __syncthreads();
    for (int ee = threadIdx.x; ee < E; ee += kPermThreads) {
      int add = 0;
      for (int w = 0; w < kPermThreads / 64; ++w) {
        add += wcnt[w][ee];
        wcnt[w][ee] = 0;
      }
      run[ee] += add;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kPermThreads) void perm_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ gates, int R, int E,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_src, int32_t* __restrict__ inv,
    float* __restrict__ row_gate) {
  __shared__ int32_t run[256];
  __shared__ int32_t wcnt[kPermThreads / 64][256];
  int ev[kRounds];
  load_chunk(ids, R, E, blockIdx.x, ev);
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    run[e] = offsets[e] + chunk_base[static_cast<size_t>(blockIdx.x) * E + e];
  }
  for (int i = threadIdx.x; i < (kPermThreads / 64) * 256; i += kPermThreads)
    (&wcnt[0][0])[i] = 0;
  __syncthreads();
  scatter_chunk(ev, gates, R, E, blockIdx.x, run, wcnt, sorted_src, inv, row_gate);
}

// All three steps in one workgroup when the flat ids fit one chunk (decode
// batches): saves two launches on the latency-bound path.
__global__ __launch_bounds__(kPermThreads) void perm_single_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ gates, int R, int E,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int bm0,
    int32_t* __restrict__ tile_off0, int bm1, int32_t* __restrict__ tile_off1,
    uint32_t* __restrict__ zero_words, int n_zero, int32_t* __restrict__ sorted_src,
    int32_t* __restrict__ inv, float* __restrict__ row_gate) {
  __shared__ int32_t cnt[256];
  __shared__ int32_t wcnt[kPermThreads / 64][256];
  __shared__ int tmp[kPermThreads / 64];
  int ev[kRounds];
  load_chunk(ids, R, E, 0, ev);
  for (int e = threadIdx.x; e < 256; e += kPermThreads) cnt[e] = 0;
  for (int i = threadIdx.x; i < (kPermThreads / 64) * 256; i += kPermThreads)
    (&wcnt[0][0])[i] = 0;
  __syncthreads();
  count_chunk(ev, cnt);
  __syncthreads();
  const int e = threadIdx.x;
  const int run = e < E ? cnt[e] : 0;
  scan_experts(run, E, counts, offsets, bm0, tile_off0, bm1, tile_off1, zero_words, n_zero, tmp);
  __syncthreads();
  // cnt[] becomes the running first row of each expert
  if (e < E) cnt[e] = offsets[e];
  __syncthreads();
  scatter_chunk(ev, gates, R, E, 0, cnt, wcnt, sorted_src, inv, row_gate);
}

// The identity permutation of one expert that takes all R rows with gate
// 1: row i is flat entry i.  Workgroup 0 also writes the counts, offsets and
// tile prefixes and clears the accumulation words.
__global__ __launch_bounds__(kPermThreads) void perm_identity_kernel(
    int R, int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int bm0,
    int32_t* __restrict__ tile_off0, int bm1, int32_t* __restrict__ tile_off1,
    uint32_t* __restrict__ zero_words, int n_zero, int32_t* __restrict__ sorted_src,
    int32_t* __restrict__ inv, float* __restrict__ row_gate) {
  for (int i = blockIdx.x * kPermThreads + threadIdx.x; i < R; i += gridDim.x * kPermThreads) {
    sorted_src[i] = i;
    inv[i] = i;
    row_gate[i] = 1.0f;
  }
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < n_zero; i += kPermThreads) zero_words[i] = 0u;
    if (threadIdx.x == 0) {
      counts[0] = R;
      offsets[0] = 0;
      offsets[1] = R;
      tile_off0[0] = 0;
      tile_off0[1] = (R + bm0 - 1) / bm0;
      tile_off1[0] = 0;
      tile_off1[1] = (R + bm1 - 1) / bm1;
    }
  }
}

}  // namespace

hipError_t launch_permute_identity(int R, const PermBufs& p, hipStream_t stream) {
  int g = (R + kPermThreads - 1) / kPermThreads;
  g = g < 1 ? 1 : (g > 1024 ? 1024 : g);
  hipLaunchKernelGGL(perm_identity_kernel, dim3(g), dim3(kPermThreads), 0, stream, R, p.counts,
                     p.offsets, p.bm0, p.tile_off0, p.bm1, p.tile_off1, p.zero_words, p.n_zero,
                     p.sorted_src, p.inv, p.row_gate);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, const float* gates, int T, int E, int k,
                          const PermBufs& p, hipStream_t stream) {
  const int R = T * k;
  const int n_chunks = (R + kChunk - 1) / kChunk;
  if (n_chunks <= 1) {
    hipLaunchKernelGGL(perm_single_kernel, dim3(1), dim3(kPermThreads), 0, stream, ids, gates, R,
                       E, p.counts, p.offsets, p.bm0, p.tile_off0, p.bm1, p.tile_off1,
                       p.zero_words, p.n_zero, p.sorted_src, p.inv, p.row_gate);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(perm_count_kernel, dim3(n_chunks), dim3(kPermThreads), 0, stream, ids, R,
                     E, p.chunk_counts);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kPermThreads), 0, stream,
                     p.chunk_counts, n_chunks, E, p.chunk_base, p.counts, p.offsets, p.bm0,
                     p.tile_off0, p.bm1, p.tile_off1, p.zero_words, p.n_zero);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(n_chunks), dim3(kPermThreads), 0, stream, ids,
                     gates, R, E, p.chunk_base, p.offsets, p.sorted_src, p.inv, p.row_gate);
  return hipGetLastError();
}

}  // namespace moe
