// C ABI of libmoe: host-side validation, workspace layout and the launch
// sequence of the routed MoE layer.  Declarations and argument contracts are
// in include/moe.h.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <limits>
#include <mutex>

#include "../../include/moe.h"

#include "moe_common.h"
#include "moe_internal.h"

namespace {

using moe::kBF16;
using moe::kFP8;
using moe::kNVFP4;

constexpr int32_t kMaxTokens = 1 << 20;
constexpr size_t kAlign = 256;
constexpr int kTileRowsMin = 32;  // smallest rows-per-tile of any GEMM shape

// MOE_EINVAL for malformed dims (null, non-positive, k > E), MOE_EUNSUPPORTED
// for well-formed shapes outside what the kernels cover.
moe_status dims_check(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->hidden <= 0 || d->ffn <= 0 || d->n_experts <= 0 || d->top_k <= 0) return MOE_EINVAL;
  if (d->top_k > d->n_experts) return MOE_EINVAL;
  if (d->hidden % 64 || d->ffn % 64) return MOE_EUNSUPPORTED;
  if (d->n_experts < 16 || d->n_experts > 256 || d->n_experts % 16) return MOE_EUNSUPPORTED;
  if (d->top_k > 8) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

bool dims_ok(const moe_dims* d) { return dims_check(d) == MOE_OK; }

// the shared expert: one expert (E = 1) that every token takes (k = 1)
moe_status shared_dims_check(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->hidden <= 0 || d->ffn <= 0 || d->n_experts != 1 || d->top_k != 1) return MOE_EINVAL;
  if (d->hidden % 64 || d->ffn % 64) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// an expert bank to pack: any expert count, layer widths as dims_check
moe_status bank_dims_check(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->hidden <= 0 || d->ffn <= 0 || d->n_experts <= 0) return MOE_EINVAL;
  if (d->hidden % 64 || d->ffn % 64 || d->n_experts > 256) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

bool fmt_ok(int32_t fmt) { return fmt == kBF16 || fmt == kFP8 || fmt == kNVFP4; }

bool aligned(const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

// The kernels move token rows, weight rows and output rows in 16-byte
// vectors and routing entries, scales and block scales as 4-byte words.
bool bank_aligned(const moe_experts* ex) {
  if (!aligned(ex->up, 16) || !aligned(ex->down, 16)) return false;
  if (ex->fmt != kBF16 && (!aligned(ex->up_s, 4) || !aligned(ex->down_s, 4))) return false;
  if (ex->fmt == kNVFP4 && (!aligned(ex->up_bs, 4) || !aligned(ex->down_bs, 4))) return false;
  return true;
}

struct Layout {
  size_t counts, offsets, scales, chunk_counts, chunk_base, tile_off0, tile_off1, sorted_src,
      inv, row_gate, act, out_rows, x_q, act_q, total;
  bool has_xq, has_actq, actq_inplace;
  int max_tiles;
};

// scales floats: [0] x scale, [1] act scale; then the amax slots of x and of
// the intermediate (kAmaxSlots words each, fp32 bits)
Layout make_layout(const moe_dims* d, int32_t fmt, int32_t T) {
  Layout L{};
  const size_t E = static_cast<size_t>(d->n_experts);
  const size_t R = static_cast<size_t>(T) * d->top_k;
  const size_t H = static_cast<size_t>(d->hidden), F = static_cast<size_t>(d->ffn);
  const size_t n_chunks = R ? (R + moe::kChunk - 1) / moe::kChunk : 1;
  const size_t max_tiles = (R + kTileRowsMin - 1) / kTileRowsMin + (R < E ? R : E) + 1;
  size_t off = 0;
  auto alloc = [&](size_t bytes) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    const size_t at = off;
    off += bytes;
    return at;
  };
  L.counts = alloc(E * 4);
  L.offsets = alloc((E + 1) * 4);
  L.scales = alloc((16 + 2 * moe::kAmaxSlots) * 4);
  L.chunk_counts = alloc(n_chunks * E * 4);
  L.chunk_base = alloc(n_chunks * E * 4);
  L.tile_off0 = alloc((E + 1) * 4);
  L.tile_off1 = alloc((E + 1) * 4);
  L.sorted_src = alloc(R * 4);
  L.inv = alloc(R * 4);
  L.row_gate = alloc(R * 4);
  L.act = alloc(R * F * 2);
  L.out_rows = alloc(R * H * 4);
  L.has_xq = fmt != kBF16;
  L.has_actq = fmt != kBF16;
  L.actq_inplace = fmt == kNVFP4;
  L.x_q = L.has_xq ? alloc(static_cast<size_t>(T) * H * 2) : 0;
  L.act_q = fmt == kFP8 ? alloc(R * F) : L.act;
  L.total = (off + kAlign - 1) / kAlign * kAlign;
  L.max_tiles = static_cast<int>(max_tiles);
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// ---- expert cache: replacement state in the caller's host buffer
constexpr uint32_t kCacheMagic = 0x4d6f4543u;

struct CacheHeader {
  uint32_t magic;
  int32_t n_experts, n_slots, fmt;
  int64_t tick;
};

// views of the state buffer: header, then slot -> expert, expert -> slot,
// last use of each expert, and host staging for the per-expert row counts
// (device to host) and the slot map (host to device)
struct CacheView {
  CacheHeader* h;
  int32_t* slot_expert;  // [n_slots], -1 = empty
  int32_t* expert_slot;  // [E], -1 = not resident
  int64_t* last_use;     // [E]
  int32_t* counts;       // [E]
  int32_t* slot_of;      // [E], the device map's host copy
};

size_t cache_state_bytes(int E, int n_slots) {
  return sizeof(CacheHeader) + static_cast<size_t>(n_slots) * 4 + static_cast<size_t>(E) * (4 + 8 + 4 + 4);
}

CacheView cache_view(void* state, int E, int n_slots) {
  uint8_t* p = static_cast<uint8_t*>(state);
  CacheView v;
  v.h = reinterpret_cast<CacheHeader*>(p);
  p += sizeof(CacheHeader);
  v.last_use = reinterpret_cast<int64_t*>(p);  // 8-byte fields first (header size is a multiple of 8)
  p += static_cast<size_t>(E) * 8;
  v.slot_expert = reinterpret_cast<int32_t*>(p);
  p += static_cast<size_t>(n_slots) * 4;
  v.expert_slot = reinterpret_cast<int32_t*>(p);
  p += static_cast<size_t>(E) * 4;
  v.counts = reinterpret_cast<int32_t*>(p);
  p += static_cast<size_t>(E) * 4;
  v.slot_of = reinterpret_cast<int32_t*>(p);
  return v;
}

// bytes of one expert's codes and (NVFP4) block scales in a projection N x K
size_t expert_code_bytes(int fmt, int N, int K) {
  const size_t n = static_cast<size_t>(N) * K;
  return fmt == kBF16 ? 2 * n : (fmt == kFP8 ? n : n / 2);
}
size_t expert_scale_bytes(int fmt, int N, int K) {
  return fmt == kNVFP4 ? static_cast<size_t>(N) * K / 16 : 0;
}

moe_status cache_check(const moe_dims* d, const moe_cache* c) {
  if (!c) return MOE_EINVAL;
  if (!fmt_ok(c->host.fmt)) return MOE_EINVAL;
  if (c->n_slots < d->top_k || c->n_slots > d->n_experts) return MOE_EINVAL;
  if (!c->host.up || !c->host.down || !c->slot_up || !c->slot_down || !c->slot_of)
    return MOE_EINVAL;
  if (c->host.fmt != kBF16 && (!c->up_s || !c->down_s)) return MOE_EINVAL;
  if (c->host.fmt == kNVFP4 &&
      (!c->host.up_bs || !c->host.down_bs || !c->slot_up_bs || !c->slot_down_bs))
    return MOE_EINVAL;
  return MOE_OK;
}

// what a cached forward needs besides forward_impl's arguments
struct CacheCall {
  const moe_cache* cache;
  void* state;
  moe_cache_stats* stats;
};

// ---- fixed device scratch of moe_forward_noalloc.  Every GPU the library
// runs on holds its own copy of this array until the process ends.  In host
// code `scratch` only names the symbol: the device address of the current
// device's copy comes from hipGetSymbolAddress, looked up once per device and
// kept in scratch_at[]; kernels receive that address, never the array's name.
constexpr size_t kNoallocScratch = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoallocScratch];
std::mutex scratch_mu;
void* scratch_at[kMaxDevices];

// device address of `scratch` on device `dev`, which must be current
moe_status scratch_for(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_at[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
    scratch_at[dev] = p;
  }
  *out = scratch_at[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int32_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or format";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

size_t moe_workspace_size(const moe_dims* dims, int32_t fmt, int32_t max_tokens) {
  if (!dims_ok(dims) || !fmt_ok(fmt) || max_tokens < 0 || max_tokens > kMaxTokens) return 0;
  return make_layout(dims, fmt, max_tokens).total;
}

int32_t moe_workspace_layout(const moe_dims* dims, int32_t fmt, int32_t T, moe_ws_layout* out) {
  if (!out || !dims_ok(dims) || !fmt_ok(fmt) || T < 0 || T > kMaxTokens) return MOE_EINVAL;
  const Layout L = make_layout(dims, fmt, T);
  out->counts = static_cast<int64_t>(L.counts);
  out->offsets = static_cast<int64_t>(L.offsets);
  out->sorted_src = static_cast<int64_t>(L.sorted_src);
  out->inv = static_cast<int64_t>(L.inv);
  out->act = static_cast<int64_t>(L.act);
  out->out_rows = static_cast<int64_t>(L.out_rows);
  out->x_q = L.has_xq ? static_cast<int64_t>(L.x_q) : -1;
  out->act_q = L.has_actq ? static_cast<int64_t>(L.act_q) : -1;
  out->scales = static_cast<int64_t>(L.scales);
  out->total = static_cast<int64_t>(L.total);
  return MOE_OK;
}

size_t moe_cache_state_size(const moe_dims* dims, int32_t n_slots) {
  if (!dims_ok(dims) || n_slots < dims->top_k || n_slots > dims->n_experts) return 0;
  return cache_state_bytes(dims->n_experts, n_slots);
}

int32_t moe_cache_init(const moe_dims* dims, const moe_cache* cache, void* state,
                       size_t state_bytes, void* stream) {
  if (const moe_status ds = dims_check(dims)) return ds;
  if (const moe_status cs = cache_check(dims, cache)) return cs;
  const int E = dims->n_experts, S = cache->n_slots;
  if (!state || state_bytes < cache_state_bytes(E, S) || reinterpret_cast<uintptr_t>(state) % 8)
    return MOE_EINVAL;
  const CacheView v = cache_view(state, E, S);
  v.h->magic = kCacheMagic;
  v.h->n_experts = E;
  v.h->n_slots = S;
  v.h->fmt = cache->host.fmt;
  v.h->tick = 0;
  for (int i = 0; i < S; ++i) v.slot_expert[i] = -1;
  for (int e = 0; e < E; ++e) {
    v.expert_slot[e] = -1;
    v.last_use[e] = -1;
    v.counts[e] = 0;
    v.slot_of[e] = -1;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(cache->slot_of, v.slot_of, static_cast<size_t>(E) * 4,
                     hipMemcpyHostToDevice, st) != hipSuccess)
    return MOE_EHIP;
  return hip_status(hipStreamSynchronize(st));
}

size_t moe_route_workspace_size(const moe_dims* dims, int32_t max_tokens) {
  if (!dims_ok(dims) || max_tokens < 0 || max_tokens > kMaxTokens) return 0;
  const int slices = std::max(moe::router_k_slices(1, dims->hidden),
                              moe::router_k_slices(1 << 20, dims->hidden));
  const size_t bytes = static_cast<size_t>(slices) * static_cast<size_t>(max_tokens) *
                       dims->n_experts * 4;
  return bytes < kAlign ? kAlign : (bytes + kAlign - 1) / kAlign * kAlign;
}

int32_t moe_router_pack(const moe_dims* dims, const float* w, void* w_packed, void* stream) {
  if (const moe_status ds = dims_check(dims)) return ds;
  if (!w || !w_packed) return MOE_EINVAL;
  return hip_status(moe::launch_router_pack(w, dims->n_experts, dims->hidden,
                                            static_cast<uint16_t*>(w_packed),
                                            static_cast<hipStream_t>(stream)));
}

int32_t moe_route(const moe_dims* dims, int32_t T, const void* x, const moe_router* router,
                  int32_t* ids, float* gates, void* ws, size_t ws_bytes, void* stream) {
  if (const moe_status ds = dims_check(dims)) return ds;
  if (T < 0 || T > kMaxTokens) return MOE_EINVAL;
  if (T == 0) return MOE_OK;  // nothing is read or written; pointers may be null
  if (!router || !router->w_packed || !x || !ids || !gates) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(router->w_packed, 16) || !aligned(router->bias, 4) ||
      !aligned(ids, 4) || !aligned(gates, 4))
    return MOE_EINVAL;
  const size_t need = static_cast<size_t>(moe::router_k_slices(T, dims->hidden)) * T *
                      dims->n_experts * 4;
  if (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_EWORKSPACE;
  return hip_status(moe::launch_router(static_cast<const uint16_t*>(x),
                                       static_cast<const uint16_t*>(router->w_packed),
                                       router->bias, T, dims->hidden, dims->n_experts,
                                       dims->top_k, static_cast<float*>(ws), ids, gates,
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// records events[stage] (if given) on the stream before each stage
struct StageMarks {
  void* const* ev;
  int n;
  hipStream_t st;
  void mark(int i) const {
    if (ev && i < n && ev[i]) (void)hipEventRecord(static_cast<hipEvent_t>(ev[i]), st);
  }
  // events that take the own start and end of GEMM launch `stage` (0 up,
  // 1 down), when the caller passed them
  moe::KernelEvents gemm(int stage) const {
    moe::KernelEvents k;
    const int i = MOE_N_STAGES + 1 + 2 * stage;
    if (ev && n >= MOE_N_STAGES + 5) {
      k.start = static_cast<hipEvent_t>(ev[i]);
      k.stop = static_cast<hipEvent_t>(ev[i + 1]);
    }
    return k;
  }
};

// The forward pass.  With `cc` set, the expert weights come from the cache:
// after the permutation the row counts go to the host, the missing experts
// are uploaded into slots, and the GEMMs read the slots through slot_of.
// With `shared`, the one expert of dims (E = 1, k = 1) takes every token with
// weight 1 (no ids or gates); with `accumulate`, the result is added to the
// fp32 values y holds.
int32_t forward_impl(const moe_dims* dims, int32_t T, const void* x, const int32_t* ids,
                     const float* gates, const moe_experts* ex_in, void* y, int32_t y_dtype,
                     void* ws, size_t ws_bytes, void* stream, void* const* events,
                     int32_t n_events, const CacheCall* cc = nullptr, bool shared = false,
                     bool accumulate = false) {
  if (const moe_status ds = shared ? shared_dims_check(dims) : dims_check(dims)) return ds;
  moe_experts cached_bank{};
  const moe_experts* ex = ex_in;
  if (cc) {
    if (const moe_status cs = cache_check(dims, cc->cache)) return cs;
    const moe_cache* c = cc->cache;
    if (!cc->state || reinterpret_cast<uintptr_t>(cc->state) % 8) return MOE_EINVAL;
    const CacheHeader* h = static_cast<const CacheHeader*>(cc->state);
    if (h->magic != kCacheMagic || h->n_experts != dims->n_experts || h->n_slots != c->n_slots ||
        h->fmt != c->host.fmt)
      return MOE_EINVAL;  // not initialised by moe_cache_init for this cache
    cached_bank.fmt = c->host.fmt;
    cached_bank.up = c->slot_up;
    cached_bank.down = c->slot_down;
    cached_bank.up_bs = c->slot_up_bs;
    cached_bank.down_bs = c->slot_down_bs;
    cached_bank.up_s = c->up_s;
    cached_bank.down_s = c->down_s;
    ex = &cached_bank;
    if (cc->stats) *cc->stats = moe_cache_stats{0, 0, 0, 0};
  }
  if (!ex) return MOE_EINVAL;
  if (T < 0 || T > kMaxTokens) return MOE_EINVAL;
  if (!fmt_ok(ex->fmt)) return MOE_EINVAL;
  if (y_dtype != MOE_Y_BF16 && y_dtype != MOE_Y_F32) return MOE_EINVAL;
  if (accumulate && y_dtype != MOE_Y_F32) return MOE_EINVAL;
  if (T == 0) return MOE_OK;  // nothing is read or written; pointers may be null
  if (!x || !y || !ex->up || !ex->down) return MOE_EINVAL;
  if (!shared && (!ids || !gates)) return MOE_EINVAL;
  if (ex->fmt != kBF16 && (!ex->up_s || !ex->down_s)) return MOE_EINVAL;
  if (ex->fmt == kNVFP4 && (!ex->up_bs || !ex->down_bs)) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ids, 4) || !aligned(gates, 4) ||
      !bank_aligned(ex))
    return MOE_EINVAL;
  const Layout L = make_layout(dims, ex->fmt, T);
  if (!ws || ws_bytes < L.total) return MOE_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_EWORKSPACE;

  const hipStream_t st = static_cast<hipStream_t>(stream);
  const StageMarks marks{events, n_events, st};
  const int fmt = ex->fmt;
  const int H = dims->hidden, F = dims->ffn, E = dims->n_experts, k = dims->top_k;
  const int R = T * k;
  float* scales = at<float>(ws, L.scales);
  uint32_t* amax_x = reinterpret_cast<uint32_t*>(scales + 16);
  uint32_t* amax_a = amax_x + moe::kAmaxSlots;
  int32_t* offsets = at<int32_t>(ws, L.offsets);

  // 1. histogram, prefix sum + tile lists, stable scatter
  moe::PermBufs p{};
  p.chunk_counts = at<int32_t>(ws, L.chunk_counts);
  p.chunk_base = at<int32_t>(ws, L.chunk_base);
  p.counts = at<int32_t>(ws, L.counts);
  p.offsets = offsets;
  p.sorted_src = at<int32_t>(ws, L.sorted_src);
  p.inv = at<int32_t>(ws, L.inv);
  p.row_gate = at<float>(ws, L.row_gate);
  p.bm0 = moe::gemm_shape(fmt, 0, T).bm;
  p.tile_off0 = at<int32_t>(ws, L.tile_off0);
  p.bm1 = moe::gemm_shape(fmt, 1, T).bm;
  p.tile_off1 = at<int32_t>(ws, L.tile_off1);
  p.zero_words = amax_x;  // amax slots of x and of the intermediate
  p.n_zero = 2 * moe::kAmaxSlots;
  marks.mark(0);
  hipError_t err = shared ? moe::launch_permute_identity(R, p, st)
                          : moe::launch_permute(ids, gates, T, E, k, p, st);
  if (err != hipSuccess) return MOE_EHIP;

  // 1b. cached weights: bring the experts this batch touches into slots
  const int32_t* w_slot = nullptr;
  if (cc) {
    const moe_cache* c = cc->cache;
    const int S = c->n_slots;
    const CacheView v = cache_view(cc->state, E, S);
    if (hipMemcpyAsync(v.counts, p.counts, static_cast<size_t>(E) * 4, hipMemcpyDeviceToHost,
                       st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return MOE_EHIP;
    int touched = 0;
    for (int e = 0; e < E; ++e) touched += v.counts[e] > 0;
    if (touched > S) return MOE_EUNSUPPORTED;
    const int64_t now = ++v.h->tick;
    int hits = 0, misses = 0;
    int64_t bytes = 0;
    const size_t up_b = expert_code_bytes(fmt, F, H), down_b = expert_code_bytes(fmt, H, F);
    const size_t up_sb = expert_scale_bytes(fmt, F, H), down_sb = expert_scale_bytes(fmt, H, F);
    for (int e = 0; e < E; ++e) {
      if (v.counts[e] <= 0) continue;
      if (v.expert_slot[e] >= 0) {
        ++hits;
        v.last_use[e] = now;
        continue;
      }
      // a free slot, else the least recently used resident expert this
      // batch does not touch (touched experts are stamped `now`)
      int slot = -1;
      int64_t oldest = now;
      for (int i = 0; i < S && slot < 0; ++i)
        if (v.slot_expert[i] < 0) slot = i;
      if (slot < 0) {
        for (int i = 0; i < S; ++i) {
          const int r = v.slot_expert[i];
          if (v.counts[r] <= 0 && v.last_use[r] < oldest) {
            oldest = v.last_use[r];
            slot = i;
          }
        }
      }
      if (slot < 0) return MOE_EHIP;  // cannot happen: touched <= S
      if (v.slot_expert[slot] >= 0) {
        v.expert_slot[v.slot_expert[slot]] = -1;
        v.slot_of[v.slot_expert[slot]] = -1;
      }
      v.slot_expert[slot] = e;
      v.expert_slot[e] = slot;
      v.slot_of[e] = slot;
      v.last_use[e] = now;
      ++misses;
      auto up_src = static_cast<const uint8_t*>(c->host.up) + static_cast<size_t>(e) * up_b;
      auto down_src = static_cast<const uint8_t*>(c->host.down) + static_cast<size_t>(e) * down_b;
      hipError_t ce = hipMemcpyAsync(static_cast<uint8_t*>(c->slot_up) + slot * up_b, up_src, up_b,
                                     hipMemcpyHostToDevice, st);
      if (ce == hipSuccess)
        ce = hipMemcpyAsync(static_cast<uint8_t*>(c->slot_down) + slot * down_b, down_src, down_b,
                            hipMemcpyHostToDevice, st);
      if (ce == hipSuccess && up_sb)
        ce = hipMemcpyAsync(c->slot_up_bs + slot * up_sb, c->host.up_bs + e * up_sb, up_sb,
                            hipMemcpyHostToDevice, st);
      if (ce == hipSuccess && down_sb)
        ce = hipMemcpyAsync(c->slot_down_bs + slot * down_sb, c->host.down_bs + e * down_sb,
                            down_sb, hipMemcpyHostToDevice, st);
      if (ce != hipSuccess) return MOE_EHIP;
      bytes += static_cast<int64_t>(up_b + down_b + up_sb + down_sb);
    }
    // the device map changes only with an upload (moe_cache_init wrote it first)
    if (misses > 0 && hipMemcpyAsync(c->slot_of, v.slot_of, static_cast<size_t>(E) * 4,
                                     hipMemcpyHostToDevice, st) != hipSuccess)
      return MOE_EHIP;
    w_slot = c->slot_of;
    if (cc->stats) *cc->stats = moe_cache_stats{touched, hits, misses, bytes};
  }

  // 2. token quantisation (fp8 / nvfp4)
  marks.mark(1);
  const void* a_up = x;
  if (fmt == kFP8 || fmt == kNVFP4) {
    err = moe::launch_quant_tensor(fmt, static_cast<const uint16_t*>(x), T, H, amax_x, 0,
                                   at<uint16_t>(ws, L.x_q), nullptr, nullptr, scales + 0, st);
    a_up = at<uint16_t>(ws, L.x_q);
  }
  if (err != hipSuccess) return MOE_EHIP;

  // 3. grouped up projection + ReLU^2
  marks.mark(2);
  moe::GemmArgs g{};
  g.tile_off = p.tile_off0;
  g.E = E;
  g.max_tiles = (R + p.bm0 - 1) / p.bm0 + (R < E ? R : E);
  g.offsets = offsets;
  g.sorted_src = p.sorted_src;
  g.top_k = k;
  g.a = a_up;
  g.b = ex->up;
  g.b_bs = ex->up_bs;
  g.b_s = ex->up_s;
  g.a_s = scales + 0;
  g.N = F;
  g.K = H;
  g.out = at<uint16_t>(ws, L.act);
  g.row_gate = nullptr;
  g.amax = amax_a;
  g.w_slot = w_slot;
  err = moe::launch_gemm(fmt, 0, T, g, st, marks.gemm(0));
  if (err != hipSuccess) return MOE_EHIP;

  // 4. intermediate quantisation (fp8 / nvfp4), rows [0, offsets[E])
  marks.mark(3);
  const void* a_down = at<uint16_t>(ws, L.act);
  if (fmt == kFP8) {
    err = moe::launch_quant_fp8(at<uint16_t>(ws, L.act), offsets + E, R, F, amax_a, 1, nullptr,
                                at<uint8_t>(ws, L.act_q), scales + 1, st);
    a_down = at<uint8_t>(ws, L.act_q);
  } else if (fmt == kNVFP4) {
    err = moe::launch_quant_nvfp4(at<uint16_t>(ws, L.act), offsets + E, R, F, amax_a, 0,
                                  at<uint16_t>(ws, L.act), nullptr, nullptr, scales + 1, st);
  }
  if (err != hipSuccess) return MOE_EHIP;

  // 5. grouped down projection, gate applied per row
  marks.mark(4);
  g.tile_off = p.tile_off1;
  g.max_tiles = (R + p.bm1 - 1) / p.bm1 + (R < E ? R : E);
  g.sorted_src = nullptr;
  g.a = a_down;
  g.b = ex->down;
  g.b_bs = ex->down_bs;
  g.b_s = ex->down_s;
  g.a_s = scales + 1;
  g.N = H;
  g.K = F;
  g.out = at<float>(ws, L.out_rows);
  g.row_gate = p.row_gate;
  g.amax = nullptr;
  err = moe::launch_gemm(fmt, 1, T, g, st, marks.gemm(1));
  if (err != hipSuccess) return MOE_EHIP;

  // 6. combine
  marks.mark(5);
  const int y_mode = accumulate ? moe::kYF32Add : (y_dtype == MOE_Y_F32 ? moe::kYF32 : moe::kYBF16);
  err = moe::launch_combine(at<float>(ws, L.out_rows), p.inv, T, k, H, y, y_mode, st);
  marks.mark(6);
  return hip_status(err);
}

}  // namespace

extern "C" {

int32_t moe_forward(const moe_dims* dims, int32_t T, const void* x, const int32_t* ids,
                    const float* gates, const moe_experts* ex, void* y, int32_t y_dtype,
                    void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(dims, T, x, ids, gates, ex, y, y_dtype, ws, ws_bytes, stream, nullptr, 0);
}

int32_t moe_forward_timed(const moe_dims* dims, int32_t T, const void* x, const int32_t* ids,
                          const float* gates, const moe_experts* ex, void* y, int32_t y_dtype,
                          void* ws, size_t ws_bytes, void* stream, void* const* events,
                          int32_t n_events) {
  if (!events || n_events < MOE_N_STAGES + 1) return MOE_EINVAL;
  return forward_impl(dims, T, x, ids, gates, ex, y, y_dtype, ws, ws_bytes, stream, events,
                      n_events);
}

size_t moe_shared_workspace_size(const moe_dims* dims, int32_t fmt, int32_t max_tokens) {
  if (shared_dims_check(dims) != MOE_OK || !fmt_ok(fmt) || max_tokens < 0 ||
      max_tokens > kMaxTokens)
    return 0;
  return make_layout(dims, fmt, max_tokens).total;
}

int32_t moe_shared_forward(const moe_dims* dims, int32_t T, const void* x,
                           const moe_experts* expert, void* y, int32_t y_dtype, int32_t accumulate,
                           void* ws, size_t ws_bytes, void* stream) {
  if (accumulate != 0 && accumulate != 1) return MOE_EINVAL;
  return forward_impl(dims, T, x, nullptr, nullptr, expert, y, y_dtype, ws, ws_bytes, stream,
                      nullptr, 0, nullptr, true, accumulate == 1);
}

int32_t moe_forward_noalloc(const moe_dims* dims, int32_t T, const void* x, const int32_t* ids,
                            const float* gates, const moe_experts* ex, void* y, int32_t y_dtype,
                            void* stream) {
  if (const moe_status ds = dims_check(dims)) return ds;
  if (!ex || T < 0 || T > kMaxTokens || !fmt_ok(ex->fmt)) return MOE_EINVAL;
  if (T == 0)  // validates the rest; nothing is enqueued
    return forward_impl(dims, T, x, ids, gates, ex, y, y_dtype, nullptr, 0, stream, nullptr, 0);
  if (make_layout(dims, ex->fmt, T).total > kNoallocScratch) return MOE_EWORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (stream) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd) != hipSuccess) return MOE_EHIP;
    if (sd != dev) return MOE_EINVAL;  // the stream's device must be the current one
  }
  void* ws = nullptr;
  if (const moe_status ss = scratch_for(dev, &ws)) return ss;
  return forward_impl(dims, T, x, ids, gates, ex, y, y_dtype, ws, kNoallocScratch, stream, nullptr,
                      0);
}

int32_t moe_forward_cached(const moe_dims* dims, int32_t T, const void* x, const int32_t* ids,
                           const float* gates, const moe_cache* cache, void* state, void* y,
                           int32_t y_dtype, void* ws, size_t ws_bytes, void* stream,
                           moe_cache_stats* stats) {
  const CacheCall cc{cache, state, stats};
  return forward_impl(dims, T, x, ids, gates, nullptr, y, y_dtype, ws, ws_bytes, stream, nullptr, 0,
                      &cc);
}

int32_t moe_quantize_experts(const moe_dims* dims, int32_t fmt, const void* up_bf16,
                             const void* down_bf16, void* up_q, void* down_q, uint8_t* up_bs,
                             uint8_t* down_bs, float* up_s, float* down_s, void* stream) {
  if (const moe_status ds = bank_dims_check(dims)) return ds;
  if (fmt != kFP8 && fmt != kNVFP4) return MOE_EINVAL;
  if (!up_bf16 || !down_bf16 || !up_q || !down_q || !up_s || !down_s) return MOE_EINVAL;
  if (fmt == kNVFP4 && (!up_bs || !down_bs)) return MOE_EINVAL;
  if (!aligned(up_bf16, 16) || !aligned(down_bf16, 16) || !aligned(up_q, 16) ||
      !aligned(down_q, 16) || !aligned(up_bs, 4) || !aligned(down_bs, 4) || !aligned(up_s, 4) ||
      !aligned(down_s, 4))
    return MOE_EINVAL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int H = dims->hidden, F = dims->ffn, E = dims->n_experts;
  hipError_t err = moe::launch_quant_weights(fmt, static_cast<const uint16_t*>(up_bf16), E, F, H,
                                             static_cast<uint8_t*>(up_q), up_bs, up_s, 0, st);
  if (err == hipSuccess)
    err = moe::launch_quant_weights(fmt, static_cast<const uint16_t*>(down_bf16), E, H, F,
                                    static_cast<uint8_t*>(down_q), down_bs, down_s, 1, st);
  return hip_status(err);
}

int32_t moe_quantize_activation(int32_t fmt, int32_t rows, int32_t cols, const void* x,
                                void* codes, uint8_t* bs, float* scale, void* ws,
                                size_t ws_bytes, void* stream) {
  if (fmt != kFP8 && fmt != kNVFP4) return MOE_EINVAL;
  if (rows < 0 || cols <= 0 || cols % 64) return MOE_EINVAL;
  if (static_cast<long long>(rows) * cols > (1ll << 31)) return MOE_EUNSUPPORTED;
  if (!x || !codes || !scale || (fmt == kNVFP4 && !bs)) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(scale, 4)) return MOE_EINVAL;
  if (!ws || ws_bytes < kAlign || !aligned(ws, 4)) return MOE_EWORKSPACE;
  if (rows == 0) return MOE_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* amax = static_cast<uint32_t*>(ws);  // kAmaxSlots words
  hipError_t err = moe::launch_zero_u32(amax, moe::kAmaxSlots, st);
  if (err == hipSuccess)
    err = moe::launch_quant_tensor(fmt, static_cast<const uint16_t*>(x), rows, cols, amax, 1,
                                   nullptr, static_cast<uint8_t*>(codes), bs, scale, st);
  return hip_status(err);
}

int32_t moe_prenorm(int32_t T, int32_t H, const void* x, void* out, void* stream) {
  if (T < 0 || T > kMaxTokens || H <= 0 || H % 64) return MOE_EINVAL;
  if (!x || !out) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(out) % 16)
    return MOE_EINVAL;  // rows move in 16-byte chunks
  if (T == 0) return MOE_OK;
  return hip_status(moe::launch_prenorm(static_cast<const uint16_t*>(x), T, H,
                                        static_cast<uint16_t*>(out),
                                        static_cast<hipStream_t>(stream)));
}

int32_t moe_residual_add(int32_t T, int32_t H, void* x, const float* y, void* stream) {
  if (T < 0 || T > kMaxTokens || H <= 0 || H % 64) return MOE_EINVAL;
  if (!x || !y) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(moe::launch_residual(static_cast<uint16_t*>(x), y, T, H,
                                         static_cast<hipStream_t>(stream)));
}

int32_t moe_residual_prenorm(int32_t T, int32_t H, void* x, const float* y, void* out,
                             void* stream) {
  if (T < 0 || T > kMaxTokens || H <= 0 || H % 64) return MOE_EINVAL;
  if (!x || !y || !out || out == x) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % 16 ||
      reinterpret_cast<uintptr_t>(out) % 16)
    return MOE_EINVAL;  // rows move in 16-byte chunks
  if (T == 0) return MOE_OK;
  return hip_status(moe::launch_residual_prenorm(static_cast<uint16_t*>(x), y, T, H,
                                                 static_cast<uint16_t*>(out),
                                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"
