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
// ballots.  No host sync.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kPermThreads = 256;
constexpr int kRounds = kChunk / kPermThreads;  // entries per thread per chunk

__global__ __launch_bounds__(kPermThreads) void perm_count_kernel(
    const int32_t* __restrict__ ids, int R, int E, int32_t* __restrict__ chunk_counts) {
  __shared__ int32_t cnt[256];
  for (int e = threadIdx.x; e < E; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int r = 0; r < kRounds; ++r) {
    const int i = base + r * kPermThreads + threadIdx.x;
    if (i < R) {
      const int e = ids[i];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  }
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

__global__ __launch_bounds__(kPermThreads) void perm_scan_kernel(
    const int32_t* __restrict__ chunk_counts, int n_chunks, int E,
    int32_t* __restrict__ chunk_base, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int bm0, int32_t* __restrict__ tile_off0, int bm1,
    int32_t* __restrict__ tile_off1, uint32_t* __restrict__ zero_words, int n_zero) {
  __shared__ int tmp[kPermThreads / 64];
  const int e = threadIdx.x;
  for (int i = threadIdx.x; i < n_zero; i += kPermThreads) zero_words[i] = 0u;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < n_chunks; ++c) {
      const size_t at = static_cast<size_t>(c) * E + e;
      chunk_base[at] = run;
      run += chunk_counts[at];
    }
    counts[e] = run;
  }
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

__global__ __launch_bounds__(kPermThreads) void perm_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ gates, int R, int E, int k,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_src, int32_t* __restrict__ inv,
    float* __restrict__ row_gate) {
  __shared__ int32_t run[256];
  __shared__ int32_t wcnt[kPermThreads / 64][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    run[e] = offsets[e] + chunk_base[static_cast<size_t>(blockIdx.x) * E + e];
  }
  for (int i = threadIdx.x; i < (kPermThreads / 64) * 256; i += kPermThreads)
    (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kRounds; ++r) {
    const int i = base + r * kPermThreads + threadIdx.x;
    int e = -1;
    if (i < R) {
      e = ids[i];
      if (e < 0 || e >= E) {
        e = -1;
        inv[i] = -1;
      }
    }
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
      row_gate[pos] = gates[i];
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

}  // namespace

hipError_t launch_permute(const int32_t* ids, const float* gates, int T, int E, int k,
                          const PermBufs& p, hipStream_t stream) {
  const int R = T * k;
  const int n_chunks = (R + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(perm_count_kernel, dim3(n_chunks), dim3(kPermThreads), 0, stream, ids, R,
                     E, p.chunk_counts);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kPermThreads), 0, stream,
                     p.chunk_counts, n_chunks, E, p.chunk_base, p.counts, p.offsets, p.bm0,
                     p.tile_off0, p.bm1, p.tile_off1, p.zero_words, p.n_zero);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(n_chunks), dim3(kPermThreads), 0, stream, ids,
                     gates, R, E, k, p.chunk_base, p.offsets, p.sorted_src, p.inv, p.row_gate);
  return hipGetLastError();
}

}  // namespace moe
