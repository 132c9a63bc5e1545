// Per-head translation and the fp32-cache translation.
//
// "Cross-Model KV Cache Transfer in Production" (pipeline stage 2) maps each
// KV head with its own d x d matrix when sender and receiver share head count
// and head dimension; stage 3 assigns each receiver layer one sender layer by
// proportional depth.  Several receiver layers may read the same sender layer
// (a deeper receiver); their workgroups run side by side on one XCD so the
// sender rows come from HBM once.  The work per byte is low (a 128 x 128 map
// per 256-byte row), so this path is bound by HBM.

#include "kvx_internal.hpp"

namespace kvx {

// ---------------------------------------------------------------- bf16 caches, d = 128
// One workgroup per (role, receiver layer l, head h, span of up to 4096
// receiver tokens; shorter spans where that fills the last round of
// workgroups) with two kinds of waves:
//   * compute waves 0..7, two per SIMD.  Wave w owns the 32 outputs
//     16s .. 16s+15 and 64+16s .. 64+16s+15 of the head (s = w mod 4), so the
//     two members (c, c+64) of every rotary pair sit in one lane
//     (accumulator elements r and r+8), and tokens 32 (w / 4) .. +31 of each
//     64-token tile: the two waves of a SIMD hold the same map rows and
//     split the tile, so one's fragment reads, epilogue and barrier wait run
//     under the other's products.  The wave's 32 rows of W_{l,h} stay in
//     registers for the whole span as MFMA A fragments (fp32 maps prepared
//     as a high and a low 16-bit half: y = x W_hi + x W_lo keeps fp32-level
//     accuracy of the map while the 16-bit inputs stay exact).
//     Sender rows of 64-token tiles stream through a ring of six 16 KB LDS
//     stages by direct global->LDS 16-byte loads that waves 0..3 issue
//     (whole 256-byte rows, 16-byte chunks XOR-swizzled by row so fragment
//     reads of 16 consecutive rows hit distinct banks); waves 4..7 issue no
//     loads and never wait on the memory counter.  The span's row indices
//     are copied to LDS once.  Keys of a rotated receiver are rotated at the
//     receiver position before rounding, with a recurrence that steps each
//     lane's (cos, sin) by 64 positions per tile from table values read
//     once.  Each tile's 64 x 128 bf16 outputs are staged in one of two
//     16 KB LDS buffers;
//   * store waves 8..11 write the staged tile one step later, 16 bytes per
//     lane and four whole 256-byte rows per instruction.
// Sender rows are bf16 cache rows (token map as row index), or, for keys
// stored rotated, fp16 rows rotated back at the sender position (run index
// as row index; the map is then prepared in fp16).  The vector-memory
// counter is per wave: compute waves only load and store waves never wait,
// so no load ever waits for stores to complete.  One barrier per tile orders
// the stages and staging buffers between the two kinds.  Workgroups are
// numbered by group of receiver layers that share a sender layer, then head,
// then layer within the group, and consecutive numbers go to one XCD: the
// 2-3 workgroups that read one sender head start together and read its rows
// through one L2, and a group's heads, which write the 256-byte pieces of the
// same receiver rows, run side by side.
constexpr int PH_TILE = 64;                      // tokens per tile
constexpr int PH_SPAN = 4096;                    // tokens per workgroup at most
constexpr int PH_MIN_SPAN = 1024;                // shortest span chosen to fill a round of workgroups
constexpr int PH_TILE_ELEMS = PH_TILE * 128;     // 16-bit elements of a tile (16 KB)
constexpr int PH_RING = 6;                       // LDS stages of sender tiles
constexpr int PH_LOADERS = 4;                    // compute waves 0..3 issue the tile loads
// NTB = 64-token tile halves (32-token blocks) per compute wave: with NTB = 1
// (every launch) eight compute waves, two per SIMD, each take one half; NTB =
// 2 would give four compute waves, each the whole tile.  Plus 4 store waves.
template <int NTB>
struct PhShape {
  static constexpr int compute = 8 / NTB;
  static constexpr int threads = 64 * (compute + 4);
};

struct HeadKArgs {
  const uint16_t* x[2];
  int64_t x_layer_stride[2];
  int32_t x_rows[2];
  const int32_t* row_of[2];
  int32_t rotate[2];
  const void* wt[2];
  const float* bias[2];
  uint16_t* out[2];
  const float2* tab_recv;
  const int64_t* slot;      // output row of each receiver token, or null (row i)
  int64_t pool_rows;        // output rows per layer
  const int32_t* recv_pos;  // rotary position of each receiver token, or null (i)
  int32_t pos_limit;
  int32_t recv_layers, recv_tokens, heads, n_span, span_len, n_blocks, xcd_remap;
  uint8_t tap[MAX_LAYERS];  // sender layer of each receiver layer
  // receiver layers form groups: maximal runs of consecutive layers with one
  // sender layer; first layer and size of each layer's group
  uint8_t gstart[MAX_LAYERS];
  uint8_t gsize[MAX_LAYERS];
};

// Physical 16-byte chunk of logical chunk c in tile row r.
__device__ __forceinline__ int ph_chunk(int r, int c) { return c ^ (r & 15); }

// Output of local row j (0..31) of compute wave w: pairs (16w + j, 64 + 16w + j).
__device__ __forceinline__ int ph_out(int w, int j) { return j < 16 ? 16 * w + j : 48 + 16 * w + j; }

struct PhTile {
  __amdgpu_buffer_rsrc_t xr;  // sender rows of layer s, head h
  const int32_t* msm;         // LDS: sender row of each token of the span
  int32_t t0, n_tok, n_tiles;
  uint32_t row_bytes;
};

// Sender rows of this lane's 4 loads of tile k (compute wave w: rows
// 16w .. 16w+15, lane j of load i takes row 16w + 4i + j/16); tiles past
// the end read an in-range entry.
struct PhRows {
  int32_t sv[4];
};
__device__ __forceinline__ PhRows ph_rows(const PhTile& pt, int k) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int32_t r0 = k * PH_TILE + 16 * wave + (lane >> 4);
  PhRows r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.sv[i] = pt.msm[min(r0 + 4 * i, PH_SPAN - 1)];
  return r;
}

// Direct loads of tile k (64 rows) into `slot` by compute wave w from its
// rows `rr`: 4 instructions of 4 rows, lane j of instruction i at physical
// chunk j%16.  Tiles past the end read nothing.
__device__ __forceinline__ void ph_issue(const PhTile& pt, int k, const PhRows& rr, uint16_t* slot) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const bool live = k < pt.n_tiles;
  const __amdgpu_buffer_rsrc_t xr = live ? pt.xr : buf_rsrc(nullptr, 0);
  const int q = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * wave + 4 * i + q;
    const uint32_t voff = static_cast<uint32_t>(rr.sv[i]) * pt.row_bytes + 16u * ph_chunk(row, lane & 15);
    dma16(xr, voff, 0, slot + (4 * wave + i) * 512);
  }
}

template <bool F16>
__device__ __forceinline__ f32x16 ph_mfma(const u32x4& w, const u32x4& x, const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, w), __builtin_bit_cast(f16x8, x), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, x), c, 0,
                                                   0, 0);
}

// Rotation state of a lane: (cos, sin) at its token(s) of the current tile
// for its 8 pairs, and the step (cos, sin)(64 t) per tile.
template <int NTB>
struct PhRot {
  float cs[NTB][8], sn[NTB][8];
  const float* step;  // LDS [2][64]: cos and sin of one tile's 64 positions for each pair
};

// Fragments of this wave's token blocks of one tile (block ti = wave / 4
// with eight compute waves, both blocks with four), MFMA D[n][tok] +=
// W[n][k] X[tok][k]; add the bias, rotate pairs when ROT, stage (bf16 nearest
// even) into `ys` as [tok][n] with swizzled chunks.  With per-token positions
// (`rpos`), the (cos, sin) of the lane's tokens (tile tokens from `tok0`) are
// read from the table instead of stepped.
// The bias comes from registers (bn) or, where registers are short (rotating
// roles with fp32 maps), from the workgroup's 128 values in LDS (bl).
template <bool WF32, bool F16, bool ROT, int NTB>
__device__ __forceinline__ void ph_compute(const uint16_t* xs, uint16_t* ys, const u32x4 (&wh)[8],
                                           const u32x4 (&wl)[8], const float (&bn)[16], const float* bl,
                                           PhRot<NTB>& rs,
                                           const int32_t* rpos, const float2* tab, int32_t tok0, int32_t n_tok_all,
                                           int32_t pos_limit) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int sw = wave & 3;
  const int tb0 = NTB == 2 ? 0 : (wave >> 2);  // first token block of this wave
  const char* xb = reinterpret_cast<const char*>(xs);
  f32x16 acc[NTB];
#pragma unroll
  for (int j = 0; j < NTB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
  // the fragments of step ks + 1 are read before the products of step ks
  // are issued, so their LDS latency runs under those products
  u32x4 xf[2][NTB];
  auto read = [&](int ks, int buf) {
#pragma unroll
    for (int j = 0; j < NTB; ++j) {
      const int row = 32 * (tb0 + j) + (lane & 31);
      xf[buf][j] = *reinterpret_cast<const u32x4*>(xb + row * 256 + 16 * ph_chunk(row, 2 * ks + (lane >> 5)));
    }
  };
  read(0, 0);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (ks < 7) {
      read(ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int b = ks & 1;
#pragma unroll
    for (int j = 0; j < NTB; ++j) acc[j] = ph_mfma<F16>(wh[ks], xf[b][j], acc[j]);
    if constexpr (WF32) {
#pragma unroll
      for (int j = 0; j < NTB; ++j) acc[j] = ph_mfma<F16>(wl[ks], xf[b][j], acc[j]);
    }
  }
  // lane: token 32 ti + lane % 32, local rows j = 8 g + 4 (lane / 32) + e
  char* yb = reinterpret_cast<char*>(ys);
#pragma unroll
  for (int j = 0; j < NTB; ++j) {
    const int ti = tb0 + j;
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      v[r] = acc[j][r] + (ROT && WF32 ? bl[ph_out(sw, 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3))] : bn[r]);
    if constexpr (ROT) {
      if (rpos) {
        int32_t pp = rpos[min(tok0 + 32 * ti + (lane & 31), n_tok_all - 1)];
        pp = pp < 0 ? 0 : (pp >= pos_limit ? pos_limit - 1 : pp);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float2 t = tab[static_cast<int64_t>(pp) * 64 + ph_out(sw, 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3))];
          const float a = v[r], b = v[r + 8];
          v[r] = a * t.x - b * t.y;
          v[r + 8] = a * t.y + b * t.x;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float a = v[r], b = v[r + 8];
          v[r] = a * rs.cs[j][r] - b * rs.sn[j][r];
          v[r + 8] = a * rs.sn[j][r] + b * rs.cs[j][r];
          const int pr = ph_out(sw, 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3));
          const float c64 = rs.step[pr], s64 = rs.step[64 + pr];
          const float cn = rs.cs[j][r] * c64 - rs.sn[j][r] * s64;
          rs.sn[j][r] = rs.sn[j][r] * c64 + rs.cs[j][r] * s64;
          rs.cs[j][r] = cn;
        }
      }
    }
    const int tok = 32 * ti + (lane & 31);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = ph_out(sw, 8 * g) >> 3;  // 16-byte chunk of outputs ph_out(s, 8g) .. +7
      const u32x2 o = u32x2{cvt_bf16x2(v[4 * g], v[4 * g + 1]), cvt_bf16x2(v[4 * g + 2], v[4 * g + 3])};
      *reinterpret_cast<u32x2*>(yb + tok * 256 + 16 * ph_chunk(tok, c) + 8 * (lane >> 5)) = o;
    }
  }
}

// Store a staged tile by the 256 threads of the store waves: thread t writes
// 16 bytes of row 16 q + t / 16 for q = 0..3 (rows past the span end are
// skipped).
// outb: row 0 of the layer and head in the output pool; tok0: the tile's
// first receiver token; slot: output row of each token (null: the token).
template <int NC>
__device__ __forceinline__ void ph_store(const uint16_t* ys, uint16_t* outb, int32_t tok0, int32_t rows,
                                         int64_t row_elems, const int64_t* slot, int64_t pool_rows) {
  const int t = threadIdx.x - 64 * NC;
  const char* yb = reinterpret_cast<const char*>(ys);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 16 * q + (t >> 4);
    const int c = t & 15;
    const u32x4 v = *reinterpret_cast<const u32x4*>(yb + row * 256 + 16 * ph_chunk(row, c));
    if (row < rows) {
      const int64_t orow = slot ? slot[tok0 + row] : static_cast<int64_t>(tok0 + row);
      // streaming store: translated rows are not read again by this kernel
      if (orow >= 0 && orow < pool_rows) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(outb + orow * row_elems + 8 * c));
    }
  }
}

__device__ __forceinline__ void ph_barrier() {
  KVX_COMPILER_FENCE();
  __builtin_amdgcn_s_barrier();
  KVX_COMPILER_FENCE();
}

// WF32: fp32 maps (prepared as two 16-bit halves); F16: fp16 sender rows
// (rotated back) and fp16 maps, else bf16; ROT: outputs rotated at the
// receiver position; NTB: token blocks per compute wave (see PhShape).
template <bool WF32, bool F16, bool ROT, int NTB>
__global__ __attribute__((amdgpu_flat_work_group_size(PhShape<NTB>::threads, PhShape<NTB>::threads),
                          amdgpu_waves_per_eu(3 - NTB / 2, 3 - NTB / 2))) void
perhead_kernel(const HeadKArgs a) {
  constexpr int NC = PhShape<NTB>::compute;
  constexpr int NT = PhShape<NTB>::threads;
  __shared__ __attribute__((aligned(1024))) uint16_t x0[PH_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t x1[PH_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t x2[PH_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t x3[PH_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t x4[PH_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t x5[PH_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t y0[PH_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t y1[PH_TILE_ELEMS];
  __shared__ int32_t msm[PH_SPAN];
  __shared__ float rot_step[2][64];
  __shared__ float bias_l[128];

  int32_t b = blockIdx.x;
  if (a.xcd_remap) b = (b & 7) * (a.n_blocks >> 3) + (b >> 3);
  // within a (role, span): group by group, head by head, the group's layers
  // innermost, so the 2-3 workgroups that read one sender head are adjacent
  const int32_t per = a.heads * a.recv_layers;
  const int32_t o = b % per;
  const int32_t span = (b / per) % a.n_span;
  const int role = (b / per) / a.n_span;
  const int32_t gs = a.gstart[o / a.heads], gz = a.gsize[o / a.heads];
  const int32_t loc = o - gs * a.heads;
  const int32_t h = loc / gz;
  const int32_t l = gs + loc % gz;
  const int32_t s = a.tap[l];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int64_t row_elems = static_cast<int64_t>(a.heads) * 128;
  const int32_t x_rows = a.x_rows[role];

  PhTile pt;
  pt.t0 = span * a.span_len;
  pt.n_tok = min(a.span_len, a.recv_tokens - pt.t0);
  pt.n_tiles = (pt.n_tok + PH_TILE - 1) / PH_TILE;
  pt.msm = msm;
  pt.row_bytes = static_cast<uint32_t>(2 * row_elems);
  const uint16_t* xs = a.x[role] + static_cast<int64_t>(s) * a.x_layer_stride[role] + h * 128;
  pt.xr = buf_rsrc(xs, static_cast<uint32_t>(static_cast<int64_t>(x_rows) * 2 * row_elems - 256 * h));
  uint16_t* outb = a.out[role] + static_cast<int64_t>(l) * a.pool_rows * row_elems + h * 128;

  // the span's sender rows, clamped to valid rows (entries past the span
  // repeat its last token)
  const int32_t* row_of = a.row_of[role];
  for (int i = threadIdx.x; i < PH_SPAN; i += NT) {
    int32_t v = row_of[pt.t0 + min(i, pt.n_tok - 1)];
    msm[i] = v < 0 ? 0 : (v >= x_rows ? x_rows - 1 : v);
  }
  if (ROT && WF32 && threadIdx.x < 128) {
    const float* bias = a.bias[role];
    bias_l[threadIdx.x] = bias ? bias[static_cast<int64_t>(l) * row_elems + h * 128 + threadIdx.x] : 0.0f;
  }
  // the rotation's step by one tile (64 positions) of each pair; the table
  // holds position 64 whenever a span has more than one tile
  if (ROT && !a.recv_pos && threadIdx.x < 64) {
    const float2 t64 = pt.n_tiles > 1 ? a.tab_recv[64 * 64 + threadIdx.x] : float2{1.0f, 0.0f};
    rot_step[0][threadIdx.x] = t64.x;
    rot_step[1][threadIdx.x] = t64.y;
  }
  __syncthreads();

  // Every wave passes the barriers B_0 .. B_n (n = n_tiles) once each: at
  // B_k tile k is in LDS and the staged tile k-1 is complete.
  if (wave >= NC) {
    ph_barrier();  // B_0
    for (int32_t k = 1; k <= pt.n_tiles; ++k) {
      ph_barrier();  // B_k: store tile k-1
      ph_store<NC>(((k - 1) & 1) ? y1 : y0, outb, pt.t0 + (k - 1) * PH_TILE, pt.n_tok - (k - 1) * PH_TILE, row_elems,
               a.slot, a.pool_rows);
    }
    return;
  }

  // compute waves.  Rotation state first (its loads precede the tile loads,
  // so waiting for them never waits for a tile): the lane's token of tile 0
  // and the step by one tile.
  const int sw = wave & 3;  // output block of this wave
  const bool loader = wave < PH_LOADERS;
  const int32_t* rpos = ROT ? a.recv_pos : nullptr;
  PhRot<NTB> rs;
  if (ROT && !rpos) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int pr = ph_out(sw, 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3));  // pair index (< 64)
#pragma unroll
      for (int j = 0; j < NTB; ++j) {
        const int ti = (NTB == 2 ? 0 : (wave >> 2)) + j;
        const int32_t tok = min(pt.t0 + 32 * ti + (lane & 31), a.recv_tokens - 1);
        const float2 t = a.tab_recv[static_cast<int64_t>(tok) * 64 + pr];
        rs.cs[j][r] = t.x;
        rs.sn[j][r] = t.y;
      }
    }
  }
  rs.step = &rot_step[0][0];

  float bn[16];
  const float* bias = a.bias[role] ? a.bias[role] + static_cast<int64_t>(l) * row_elems + h * 128 : nullptr;
  if constexpr (ROT && WF32) {
#pragma unroll
    for (int r = 0; r < 16; ++r) bn[r] = 0.0f;
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      bn[r] = bias ? bias[ph_out(sw, 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3))] : 0.0f;
  }

  // A fragments: rows n = ph_out(s, lane % 32) of W_{l,h}, prepared
  // output-major in the operand type: [n][c] (16-bit maps) or [n][hi c | lo c]
  // (fp32 maps split into halves), k = 16 ks + 8 (lane / 32) .. +8.  The map
  // loads are issued before the tiles' loads: one wait covers them (the
  // counter completes in order), and the tiles are in flight meanwhile.
  u32x4 wh[8], wl[8];
  {
    constexpr int KW = WF32 ? 256 : 128;  // 16-bit elements per map row
    const int n_row = ph_out(sw, lane & 31);
    const uint16_t* wp = static_cast<const uint16_t*>(a.wt[role]) +
                         ((static_cast<int64_t>(l) * a.heads + h) * 128 + n_row) * KW + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      wh[ks] = *reinterpret_cast<const u32x4*>(wp + 16 * ks);
      wl[ks] = WF32 ? *reinterpret_cast<const u32x4*>(wp + 128 + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (loader) {
    ph_issue(pt, 0, ph_rows(pt, 0), x0);
    ph_issue(pt, 1, ph_rows(pt, 1), x1);
    ph_issue(pt, 2, ph_rows(pt, 2), x2);
    ph_issue(pt, 3, ph_rows(pt, 3), x3);
    ph_issue(pt, 4, ph_rows(pt, 4), x4);
  }
  __builtin_amdgcn_sched_barrier(0);
  // rows of the tile the first step issues, read a step ahead from then on
  // (loading waves only)
  PhRows rr{};
  if (loader) rr = ph_rows(pt, PH_RING - 1);

  // Step k (tile k in stage k % 6, staging k % 2): a loading wave's wait
  // leaves the four younger tiles in flight, every wave's LDS wait completes
  // its staging writes, then B_k; a loading wave issues tile k+5 into the
  // stage of tile k-1, and tile k is multiplied into its staging buffer.
  // Steps past n_tiles (the unrolled loop runs a multiple of 6) pass no
  // barrier.
#define PH_STEP(K, XS, YS, XNEXT)                                              \
  {                                                                            \
    if ((K) <= pt.n_tiles) {                                                   \
      if (loader) KVX_WAIT_VM(4 * (PH_RING - 2));                              \
      KVX_WAIT_LGKM0();                                                        \
      ph_barrier();                                                            \
    }                                                                          \
    if (loader) {                                                              \
      ph_issue(pt, (K) + PH_RING - 1, rr, XNEXT);                              \
      rr = ph_rows(pt, (K) + PH_RING);                                         \
    }                                                                          \
    if ((K) < pt.n_tiles)                                                      \
      ph_compute<WF32, F16, ROT, NTB>(XS, YS, wh, wl, bn, bias_l, rs, rpos, a.tab_recv, \
                            pt.t0 + (K) * PH_TILE, a.recv_tokens, a.pos_limit); \
  }
  for (int32_t k = 0; k < pt.n_tiles; k += 6) {
    PH_STEP(k, x0, y0, x5)
    PH_STEP(k + 1, x1, y1, x0)
    PH_STEP(k + 2, x2, y0, x1)
    PH_STEP(k + 3, x3, y1, x2)
    PH_STEP(k + 4, x4, y0, x3)
    PH_STEP(k + 5, x5, y1, x4)
  }
#undef PH_STEP
  // B_n when the loop ended exactly at step n - 1; then drain the loads of
  // tiles past the end before the workgroup's LDS is released
  if (pt.n_tiles % 6 == 0) {
    KVX_WAIT_LGKM0();
    ph_barrier();
  }
  KVX_WAIT_VM(0);
}

template <bool WF32, bool F16, bool ROT>
static void ph_launch(unsigned g, const HeadKArgs& a, hipStream_t s) {
  // eight compute waves (two per SIMD, each a 32-token half of every tile);
  // rotating roles with fp32 maps read their bias and the rotation's step
  // from LDS so they fit the registers of three waves per SIMD
  constexpr int NTB = 1;
  perhead_kernel<WF32, F16, ROT, NTB><<<g, PhShape<NTB>::threads, 0, s>>>(a);
}

int launch_perhead(const HeadProblem& p, const HeadRole* roles, int n_roles, hipStream_t s) {
  if (p.recv_tokens <= 0 || n_roles <= 0) return KVX_OK;
  // one launch per operand type (fp16 rotated-back key rows, bf16 otherwise)
  // and rotation of the outputs
  for (int kind = 3; kind >= 0; --kind) {
    const int f16 = kind >> 1, rot = kind & 1;
    HeadKArgs a{};
    int n = 0;
    for (int i = 0; i < n_roles; ++i) {
      if (roles[i].x_f16 != f16 || (roles[i].rotate != 0) != (rot != 0)) continue;
      // sender rows of one layer are addressed with 32-bit byte offsets
      if (static_cast<int64_t>(roles[i].x_rows) * p.heads * 256 >= (1LL << 31)) return KVX_ERR_UNSUPPORTED;
      a.x[n] = roles[i].x;
      a.x_layer_stride[n] = roles[i].x_layer_stride;
      a.x_rows[n] = roles[i].x_rows;
      a.row_of[n] = roles[i].row_of;
      a.rotate[n] = roles[i].rotate;
      a.wt[n] = roles[i].wt;
      a.bias[n] = roles[i].bias;
      a.out[n] = roles[i].out;
      ++n;
    }
    if (n == 0) continue;
    a.tab_recv = p.tab_recv;
    a.slot = p.slot;
    a.pool_rows = p.pool_rows;
    a.recv_pos = p.recv_pos;
    a.pos_limit = p.pos_limit;
    a.recv_layers = p.recv_layers;
    a.recv_tokens = p.recv_tokens;
    a.heads = p.heads;
    // spans of up to PH_SPAN tokens; more (shorter, at least PH_MIN_SPAN)
    // spans when that fills the last round of workgroups clearly better (one
    // role per launch leaves half a round idle where two roles fill it)
    const int64_t per_span = static_cast<int64_t>(n) * p.heads * p.recv_layers;
    const int cus = device_cu_count();
    auto fill = [&](int64_t items) {
      return static_cast<double>(items) / static_cast<double>(ceil_div(items, cus) * cus);
    };
    int32_t span_len = PH_SPAN;
    double best = fill(per_span * ceil_div(p.recv_tokens, PH_SPAN));
    for (int64_t ns = ceil_div(p.recv_tokens, PH_SPAN) + 1;; ++ns) {
      const int32_t len = static_cast<int32_t>(ceil_div(ceil_div(p.recv_tokens, ns), PH_TILE) * PH_TILE);
      if (len < PH_MIN_SPAN) break;
      const double f = fill(per_span * ceil_div(p.recv_tokens, len));
      if (f > best + 0.05) {
        best = f;
        span_len = len;
      }
    }
    a.span_len = span_len;
    a.n_span = static_cast<int32_t>(ceil_div(p.recv_tokens, span_len));
    for (int l = 0; l < p.recv_layers; ++l) a.tap[l] = static_cast<uint8_t>(p.taps[l]);
    for (int l = 0; l < p.recv_layers;) {
      int e = l + 1;
      while (e < p.recv_layers && p.taps[e] == p.taps[l]) ++e;
      for (int i = l; i < e; ++i) {
        a.gstart[i] = static_cast<uint8_t>(l);
        a.gsize[i] = static_cast<uint8_t>(e - l);
      }
      l = e;
    }
    const int64_t nb = per_span * a.n_span;
    if (nb >= (1LL << 31)) return KVX_ERR_UNSUPPORTED;
    a.n_blocks = static_cast<int32_t>(nb);
    a.xcd_remap = (nb % 8 == 0) ? 1 : 0;
    const unsigned g = static_cast<unsigned>(nb);
    if (p.w_f32) {
      if (f16)
        rot ? ph_launch<true, true, true>(g, a, s) : ph_launch<true, true, false>(g, a, s);
      else
        rot ? ph_launch<true, false, true>(g, a, s) : ph_launch<true, false, false>(g, a, s);
    } else {
      if (f16)
        rot ? ph_launch<false, true, true>(g, a, s) : ph_launch<false, true, false>(g, a, s);
      else
        rot ? ph_launch<false, false, true>(g, a, s) : ph_launch<false, false, false>(g, a, s);
    }
    KVX_LAUNCH_CHECK();
  }
  return KVX_OK;
}

// ---------------------------------------------------------------- fp32 caches (any shape)
// One block per (receiver token, receiver layer, role): the feature row is
// assembled in LDS (rotated back when the sender keys are rotated), every
// output is a dot product in fp32, then outputs are rotated in pairs at the
// receiver position when the receiver keys are rotated.
constexpr int F32_MAX_FIN = 8192;

struct F32KArgs {
  const float* x[2];
  const void* wt[2];
  const float* bias[2];
  float* out[2];
  int32_t derotate[2], rotate[2];
  const int32_t* map;
  const float2* tab_send;
  const float2* tab_recv;
  int32_t send_tokens, send_heads, send_dim, recv_tokens, recv_heads, recv_dim;
  int32_t n_taps, per_head, w_f32;
  uint8_t taps[MAX_LAYERS * MAX_TAPS];
};

__global__ __launch_bounds__(256) void f32_kernel(const F32KArgs a, int64_t send_layer_stride) {
  __shared__ float xs[F32_MAX_FIN];
  __shared__ float ys[F32_MAX_FIN];
  const int32_t rho = blockIdx.x;
  const int32_t l = blockIdx.y;
  const int role = blockIdx.z;
  int32_t j = a.map[rho];
  j = j < 0 ? 0 : (j >= a.send_tokens ? a.send_tokens - 1 : j);
  const int32_t row = a.send_heads * a.send_dim;
  const int32_t shalf = a.send_dim / 2;
  const bool dr = a.derotate[role] != 0;
  for (int t = 0; t < a.n_taps; ++t) {
    const float* src = a.x[role] + a.taps[l * MAX_TAPS + t] * send_layer_stride + static_cast<int64_t>(j) * row;
    for (int e = threadIdx.x; e < row; e += blockDim.x) {
      float v = src[e];
      if (dr) {
        const int c = e % a.send_dim;
        const int hb = e - c;
        const int jj = c % shalf;
        const float2 cs = a.tab_send[static_cast<int64_t>(j) * shalf + jj];
        const float xa = src[hb + jj], xb = src[hb + jj + shalf];
        v = (c < shalf) ? (xa * cs.x + xb * cs.y) : (xb * cs.x - xa * cs.y);
      }
      xs[t * row + e] = v;
    }
  }
  __syncthreads();
  const int32_t f_out = a.recv_heads * a.recv_dim;
  const int32_t f_in = a.n_taps * row;
  const float* bias = a.bias[role] ? a.bias[role] + static_cast<int64_t>(l) * f_out : nullptr;
  for (int o = threadIdx.x; o < f_out; o += blockDim.x) {
    float acc = 0.0f;
    if (a.per_head) {
      const int h = o / a.recv_dim, c = o % a.recv_dim;
      const int64_t wrow = ((static_cast<int64_t>(l) * a.recv_heads + h) * a.recv_dim + c) * a.recv_dim;
      for (int k = 0; k < a.recv_dim; ++k) {
        const float w = a.w_f32 ? static_cast<const float*>(a.wt[role])[wrow + k]
                                : bf16_to_f32(static_cast<const uint16_t*>(a.wt[role])[wrow + k]);
        acc = fmaf(xs[h * a.recv_dim + k], w, acc);
      }
    } else {
      const int64_t wrow = (static_cast<int64_t>(l) * f_out + o) * f_in;
      for (int k = 0; k < f_in; ++k) {
        const float w = a.w_f32 ? static_cast<const float*>(a.wt[role])[wrow + k]
                                : bf16_to_f32(static_cast<const uint16_t*>(a.wt[role])[wrow + k]);
        acc = fmaf(xs[k], w, acc);
      }
    }
    ys[o] = acc + (bias ? bias[o] : 0.0f);
  }
  __syncthreads();
  float* dst = a.out[role] + (static_cast<int64_t>(l) * a.recv_tokens + rho) * f_out;
  const int32_t rhalf = a.recv_dim / 2;
  const bool rr = a.rotate[role] != 0;
  for (int o = threadIdx.x; o < f_out; o += blockDim.x) {
    float v = ys[o];
    if (rr) {
      const int c = o % a.recv_dim;
      const int hb = o - c;
      const int jj = c % rhalf;
      const float2 cs = a.tab_recv[static_cast<int64_t>(rho) * rhalf + jj];
      const float ya = ys[hb + jj], yb = ys[hb + jj + rhalf];
      v = (c < rhalf) ? (ya * cs.x - yb * cs.y) : (ya * cs.y + yb * cs.x);
    }
    dst[o] = v;
  }
}

int launch_f32(const F32Problem& p, const F32Role* roles, int n_roles, hipStream_t s) {
  if (p.recv_tokens <= 0 || n_roles <= 0) return KVX_OK;
  const int64_t f_in = static_cast<int64_t>(p.n_taps) * p.send_heads * p.send_dim;
  const int64_t f_out = static_cast<int64_t>(p.recv_heads) * p.recv_dim;
  if (f_in > F32_MAX_FIN || f_out > F32_MAX_FIN) return KVX_ERR_UNSUPPORTED;
  F32KArgs a{};
  for (int i = 0; i < n_roles; ++i) {
    a.x[i] = roles[i].x;
    a.wt[i] = roles[i].wt;
    a.bias[i] = roles[i].bias;
    a.out[i] = roles[i].out;
    a.derotate[i] = roles[i].derotate;
    a.rotate[i] = roles[i].rotate;
  }
  a.map = p.recv_to_send;
  a.tab_send = p.tab_send;
  a.tab_recv = p.tab_recv;
  a.send_tokens = p.send_tokens;
  a.send_heads = p.send_heads;
  a.send_dim = p.send_dim;
  a.recv_tokens = p.recv_tokens;
  a.recv_heads = p.recv_heads;
  a.recv_dim = p.recv_dim;
  a.n_taps = p.n_taps;
  a.per_head = p.per_head;
  a.w_f32 = p.w_f32;
  for (int l = 0; l < p.recv_layers; ++l)
    for (int t = 0; t < p.n_taps; ++t) a.taps[l * MAX_TAPS + t] = static_cast<uint8_t>(p.taps[l * p.n_taps + t]);
  const int64_t stride = static_cast<int64_t>(p.send_tokens) * p.send_heads * p.send_dim;
  dim3 grid(static_cast<unsigned>(p.recv_tokens), static_cast<unsigned>(p.recv_layers), static_cast<unsigned>(n_roles));
  f32_kernel<<<grid, 256, 0, s>>>(a, stride);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

}  // namespace kvx
