// Token alignment and run compaction.
//
// Alignment follows "Prefill-Free Cross-Family KV Cache Transfer for
// Heterogeneous Multi-Agent LLMs" (Key Contributions 1, Methodology 1):
// receiver and sender tokens are paired where they end at the same
// character; a receiver token whose end is not shared reuses the sender token
// of the latest preceding shared boundary; many-to-one takes the sender token
// at the matched boundary (no averaging).
//
// On the device this is two steps: a binary search of every receiver end in
// the sender ends (a match gives the sender index, otherwise -1), then an
// inclusive max-scan along the receiver tokens.  The matched sender indices
// increase with the receiver index, so the running maximum is exactly the
// sender token of the latest shared boundary at or before each receiver end.
// Tokens before the first shared boundary keep -1 and are set to 0.
//
// Run compaction restructures a token map into maximal runs of equal
// consecutive values (receiver tokens in one run reuse the same sender
// state): uniq[u] = value of run u, run_begin[u] = first receiver row of run
// u (run_begin[U] = N), recv_to_uniq[i] = run of row i, and U.

#include <mutex>
#include <vector>

#include "kvx_align.hpp"

namespace kvx {

constexpr int SCAN_THREADS = 256;
constexpr int SCAN_ITEMS = 4;
constexpr int SCAN_TILE = SCAN_THREADS * SCAN_ITEMS;

struct OpMax {
  static __device__ __forceinline__ int32_t apply(int32_t a, int32_t b) { return a > b ? a : b; }
  static constexpr int32_t identity = INT32_MIN;
};
struct OpSum {
  static __device__ __forceinline__ int32_t apply(int32_t a, int32_t b) { return a + b; }
  static constexpr int32_t identity = 0;
};

// Scan of one value per thread over a 256-thread block: inclusive and
// exclusive prefixes of this thread and the block aggregate.
template <class Op>
__device__ __forceinline__ void block_scan(int32_t v, int32_t* lds_waves, int32_t& incl,
                                           int32_t& excl, int32_t& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(x, d, 64);
    if (lane >= d) x = Op::apply(x, o);
  }
  int32_t xw = __shfl_up(x, 1, 64);
  if (lane == 0) xw = Op::identity;
  if (lane == 63) lds_waves[wave] = x;
  __syncthreads();
  int32_t carry = Op::identity, all = Op::identity;
  for (int w = 0; w < SCAN_THREADS / 64; ++w) {
    if (w < wave) carry = Op::apply(carry, lds_waves[w]);
    all = Op::apply(all, lds_waves[w]);
  }
  __syncthreads();
  incl = Op::apply(carry, x);
  excl = Op::apply(carry, xw);
  total = all;
}

// Phase 1: local inclusive scan of one 1024-element tile, aggregate per tile.
template <class Op>
__device__ __forceinline__ void scan_tile_local(int32_t* vals, int64_t n, int32_t* agg) {
  __shared__ int32_t lds[SCAN_THREADS / 64];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * SCAN_TILE + threadIdx.x * SCAN_ITEMS;
  int32_t v[SCAN_ITEMS];
  int32_t run = Op::identity;
#pragma unroll
  for (int k = 0; k < SCAN_ITEMS; ++k) {
    v[k] = (base + k < n) ? vals[base + k] : Op::identity;
    run = Op::apply(run, v[k]);
    v[k] = run;
  }
  int32_t incl, excl, total;
  block_scan<Op>(run, lds, incl, excl, total);
#pragma unroll
  for (int k = 0; k < SCAN_ITEMS; ++k)
    if (base + k < n) vals[base + k] = Op::apply(excl, v[k]);
  if (threadIdx.x == 0) agg[blockIdx.x] = total;
}

// Phase 2: one block turns the tile aggregates into exclusive tile carries.
template <class Op>
__global__ __launch_bounds__(SCAN_THREADS) void scan_carries(int32_t* agg, int32_t n_tiles) {
  __shared__ int32_t lds[SCAN_THREADS / 64];
  int32_t carry = Op::identity;
  for (int32_t b0 = 0; b0 < n_tiles; b0 += SCAN_THREADS) {
    const int32_t i = b0 + threadIdx.x;
    const int32_t v = (i < n_tiles) ? agg[i] : Op::identity;
    int32_t incl, excl, total;
    block_scan<Op>(v, lds, incl, excl, total);
    if (i < n_tiles) agg[i] = Op::apply(carry, excl);
    carry = Op::apply(carry, total);
  }
}

__global__ void fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

int launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return KVX_OK;
  const int64_t blocks = ceil_div(n, 256) < 1024 ? ceil_div(n, 256) : 1024;
  fill_i32<<<static_cast<unsigned>(blocks), 256, 0, s>>>(p, n, v);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// ---------------------------------------------------------------- alignment

__global__ __launch_bounds__(SCAN_THREADS) void align_match_scan(
    const int32_t* __restrict__ send_end, int32_t n_send, const int32_t* __restrict__ recv_end,
    int32_t n_recv, int32_t* __restrict__ out, int32_t* __restrict__ agg, int32_t* __restrict__ bad) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * SCAN_TILE + threadIdx.x * SCAN_ITEMS;
  // validity of the sender offsets (strictly increasing, > 0): the grid
  // covers n_recv; sender entries beyond it are checked by a grid-stride loop
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * SCAN_THREADS + threadIdx.x; j < n_send;
       j += static_cast<int64_t>(gridDim.x) * SCAN_THREADS) {
    const int32_t e = send_end[j];
    if (e <= 0 || (j > 0 && e <= send_end[j - 1])) *bad = 1;
  }
#pragma unroll
  for (int k = 0; k < SCAN_ITEMS; ++k) {
    const int64_t i = base + k;
    if (i >= n_recv) break;
    const int32_t e = recv_end[i];
    if (e <= 0 || (i > 0 && e <= recv_end[i - 1])) *bad = 1;
    // lower bound of e in send_end
    int32_t lo = 0, hi = n_send;
    while (lo < hi) {
      const int32_t mid = (lo + hi) >> 1;
      if (send_end[mid] < e) lo = mid + 1; else hi = mid;
    }
    out[i] = (lo < n_send && send_end[lo] == e) ? lo : -1;
  }
  __syncthreads();
  scan_tile_local<OpMax>(out, n_recv, agg);
}

// `add`: the sequence's first token in a concatenation of sender sequences.
__global__ __launch_bounds__(SCAN_THREADS) void align_finish(int32_t* __restrict__ out, int32_t n,
                                                             const int32_t* __restrict__ carry, int32_t add) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * SCAN_TILE + threadIdx.x * SCAN_ITEMS;
  const int32_t c = carry[blockIdx.x];
#pragma unroll
  for (int k = 0; k < SCAN_ITEMS; ++k) {
    const int64_t i = base + k;
    if (i < n) {
      const int32_t v = OpMax::apply(c, out[i]);
      out[i] = (v < 0 ? 0 : v) + add;
    }
  }
}

size_t align_ws_bytes(int32_t n_recv) {
  const int32_t ro[2] = {0, n_recv > 0 ? n_recv : 1};
  return align_batched_ws_bytes(ro, 1);
}

// One sequence, no synchronisation: flags invalid offsets in *bad.
static int align_one(const int32_t* send_end, int32_t n_send, const int32_t* recv_end, int32_t n_recv, int32_t* out,
                     int32_t add, int32_t* agg, int32_t* bad, hipStream_t s) {
  const int32_t tiles = static_cast<int32_t>(ceil_div(n_recv, SCAN_TILE));
  align_match_scan<<<tiles, SCAN_THREADS, 0, s>>>(send_end, n_send, recv_end, n_recv, out, agg, bad);
  KVX_LAUNCH_CHECK();
  scan_carries<OpMax><<<1, SCAN_THREADS, 0, s>>>(agg, tiles);
  KVX_LAUNCH_CHECK();
  align_finish<<<tiles, SCAN_THREADS, 0, s>>>(out, n_recv, agg, add);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

int launch_align(const int32_t* send_end, int32_t n_send, const int32_t* recv_end, int32_t n_recv,
                 int32_t* out, void* ws, hipStream_t s) {
  const int32_t so[2] = {0, n_send}, ro[2] = {0, n_recv};
  return launch_align_batched(send_end, so, recv_end, ro, 1, out, ws, s);
}

// One sequence without synchronisation: invalid (device) receives 1 when an
// offset array is not positive and strictly increasing, else 0.
int launch_align_async(const int32_t* send_end, int32_t n_send, const int32_t* recv_end, int32_t n_recv,
                       int32_t* out, int32_t* invalid, void* ws, hipStream_t s) {
  Carve c(ws);
  (void)c.take<int32_t>(64);  // same layout as the synchronous call
  int32_t* agg = c.take<int32_t>(ceil_div(n_recv > 0 ? n_recv : 1, SCAN_TILE));
  if (int st = launch_fill_i32(invalid, 1, 0, s)) return st;
  return align_one(send_end, n_send, recv_end, n_recv, out, 0, agg, invalid, s);
}

// ---------------------------------------------------------------- alignment without allocation
// The scan's tile aggregates of the no-allocation entry live in a file-scope
// device array.  Each device holds its own copy at its own address, found
// once per device with hipGetSymbolAddress; host code never passes the
// array's name itself (a host-side stand-in) to a kernel.  Every call on a
// device shares that device's copy: calls that overlap on one device race.
// The aggregates are written in full by the first kernel of each call before
// they are read, so nothing needs clearing between calls.
static __device__ __align__(256) int32_t scratch[NOALLOC_MAX_RECV / SCAN_TILE];

static int scratch_ptr(int32_t** out) {
  static std::mutex mu;
  static int32_t* ptr[64] = {nullptr};
  int dev = -1;
  KVX_HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return KVX_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    KVX_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return KVX_ERR_HIP;
    ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = ptr[dev];
  return KVX_OK;
}

int launch_align_noalloc(const int32_t* send_end, int32_t n_send, const int32_t* recv_end, int32_t n_recv,
                         int32_t* out, int32_t* invalid, hipStream_t s) {
  if (n_recv > NOALLOC_MAX_RECV) return KVX_ERR_WORKSPACE;
  int32_t* agg = nullptr;
  if (int st = scratch_ptr(&agg)) return st;
  if (int st = launch_fill_i32(invalid, 1, 0, s)) return st;
  return align_one(send_end, n_send, recv_end, n_recv, out, 0, agg, invalid, s);
}

size_t align_batched_ws_bytes(const int32_t* recv_off, int32_t n_seq) {
  int32_t longest = 1;
  for (int32_t q = 0; q < n_seq; ++q) longest = max(longest, recv_off[q + 1] - recv_off[q]);
  return align_up(sizeof(int32_t) * (static_cast<size_t>(n_seq) + 64), 256) +
         align_up(sizeof(int32_t) * ceil_div(longest, SCAN_TILE), 256);
}

int launch_align_batched(const int32_t* send_end, const int32_t* send_off, const int32_t* recv_end,
                         const int32_t* recv_off, int32_t n_seq, int32_t* out, void* ws, hipStream_t s) {
  Carve c(ws);
  int32_t* bad = c.take<int32_t>(static_cast<size_t>(n_seq) + 64);
  int32_t longest = 1;
  for (int32_t q = 0; q < n_seq; ++q) longest = max(longest, recv_off[q + 1] - recv_off[q]);
  int32_t* agg = c.take<int32_t>(ceil_div(longest, SCAN_TILE));  // reused in stream order
  if (int st = launch_fill_i32(bad, n_seq, 0, s)) return st;
  for (int32_t q = 0; q < n_seq; ++q) {
    const int32_t nr = recv_off[q + 1] - recv_off[q];
    if (nr == 0) continue;
    if (int st = align_one(send_end + send_off[q], send_off[q + 1] - send_off[q], recv_end + recv_off[q], nr,
                           out + recv_off[q], send_off[q], agg, bad + q, s))
      return st;
  }
  std::vector<int32_t> host_bad(static_cast<size_t>(n_seq), 0);
  KVX_HIP_TRY(hipMemcpyAsync(host_bad.data(), bad, sizeof(int32_t) * n_seq, hipMemcpyDeviceToHost, s));
  KVX_HIP_TRY(hipStreamSynchronize(s));
  for (int32_t q = 0; q < n_seq; ++q)
    if (host_bad[q]) return KVX_ERR_INVALID;
  return KVX_OK;
}

// ---------------------------------------------------------------- run compaction

__device__ __forceinline__ int32_t clamp_idx(int32_t v, int32_t n) {
  return v < 0 ? 0 : (v >= n ? n - 1 : v);
}

__global__ __launch_bounds__(SCAN_THREADS) void runs_flags_scan(
    const int32_t* __restrict__ map, int32_t n, int32_t n_send, int32_t* __restrict__ r2u,
    int32_t* __restrict__ agg) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * SCAN_TILE + threadIdx.x * SCAN_ITEMS;
#pragma unroll
  for (int k = 0; k < SCAN_ITEMS; ++k) {
    const int64_t i = base + k;
    if (i >= n) break;
    const int32_t v = clamp_idx(map[i], n_send);
    r2u[i] = (i == 0 || clamp_idx(map[i - 1], n_send) != v) ? 1 : 0;
  }
  __syncthreads();
  scan_tile_local<OpSum>(r2u, n, agg);
}

__global__ __launch_bounds__(SCAN_THREADS) void runs_finish(
    const int32_t* __restrict__ map, int32_t n, int32_t n_send, int32_t* __restrict__ r2u,
    const int32_t* __restrict__ carry, int32_t* __restrict__ uniq, int32_t* __restrict__ run_begin,
    int32_t* __restrict__ n_uniq) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * SCAN_TILE + threadIdx.x * SCAN_ITEMS;
  const int32_t c = carry[blockIdx.x];
#pragma unroll
  for (int k = 0; k < SCAN_ITEMS; ++k) {
    const int64_t i = base + k;
    if (i >= n) break;
    const int32_t u = c + r2u[i] - 1;
    r2u[i] = u;
    const int32_t v = clamp_idx(map[i], n_send);
    if (i == 0 || clamp_idx(map[i - 1], n_send) != v) {
      uniq[u] = v;
      run_begin[u] = static_cast<int32_t>(i);
    }
    if (i == n - 1) {
      *n_uniq = u + 1;
      run_begin[u + 1] = n;
    }
  }
}

size_t runs_ws_bytes(int32_t n) {
  const int64_t tiles = ceil_div(n > 0 ? n : 1, SCAN_TILE);
  return align_up(sizeof(int32_t) * tiles, 256);
}

int launch_runs(const int32_t* map, int32_t n, int32_t n_send, Runs r, void* ws, hipStream_t s) {
  if (n <= 0) {
    if (int st = launch_fill_i32(r.n_uniq, 1, 0, s)) return st;
    return launch_fill_i32(r.run_begin, 1, 0, s);
  }
  Carve c(ws);
  const int32_t tiles = static_cast<int32_t>(ceil_div(n, SCAN_TILE));
  int32_t* agg = c.take<int32_t>(tiles);
  runs_flags_scan<<<tiles, SCAN_THREADS, 0, s>>>(map, n, n_send, r.recv_to_uniq, agg);
  KVX_LAUNCH_CHECK();
  scan_carries<OpSum><<<1, SCAN_THREADS, 0, s>>>(agg, tiles);
  KVX_LAUNCH_CHECK();
  runs_finish<<<tiles, SCAN_THREADS, 0, s>>>(map, n, n_send, r.recv_to_uniq, agg, r.uniq,
                                             r.run_begin, r.n_uniq);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

}  // namespace kvx
