// Closed-form ridge fit.
//
// "Cross-Model KV Cache Transfer in Production" (pipeline stage 2) fits each
// map in closed form, W = (X^T X + lambda I)^-1 X^T Y, and "Implementation
// Guidelines" puts lambda in [1e-4, 1e-2].  Here:
//   1. G = X^T X (upper triangle) and C = X^T Y are accumulated over the
//      calibration rows on matrix cores (bf16 inputs, fp32 accumulation), the
//      rows split into S ranges whose fp32 partial sums are added in fp64
//      (fp32 inputs use an fp64-accumulated vector kernel instead);
//   2. optional centring for an unpenalised intercept, lambda from the trace,
//      lambda added to the diagonal (fp64, on the device);
//   3. blocked Cholesky G + lambda I = L L^T in fp64 (64-wide blocks: diagonal
//      factor and its inverse by one wave, panel triangular solve and
//      trailing update as fp64 matrix-core products), then L Z = C and
//      L^T W = Z by 256-row blocks with the inverses of the 256-wide
//      diagonal blocks (assembled from the 64-wide ones by block
//      substitution), so the right-hand sides are read and written 12
//      rather than 48 times;
//   4. W written output-major in fp32, b = mean_y - mean_x W.
// Several problems of one shape (the maps of every layer and role) are
// fitted by one call: steps 1, 2 and 4 run problem by problem (each fills
// the GPU), step 3 runs every launch of its serial chain over all problems
// at once, so the chain's latency is paid once per call.  A non-positive
// pivot sets the problem's device flag; the host reads the flags once.

#include <algorithm>
#include <array>
#include <cmath>
#include <map>
#include <vector>

#include "kvx_fit.hpp"

namespace kvx {

constexpr int GR_T = 256;          // Gram tile (features x features)
constexpr int GR_BK = 64;          // rows per K step
constexpr int GR_MAX_SPLIT = 8;
constexpr int GR_THREADS = 512;    // 8 waves, two per SIMD
constexpr int GR_PART = GR_BK * GR_T;  // 16-bit elements of one ring part (32 KB)
constexpr int GR_LD = 4;           // direct loads (1 KB each) per wave per part and step
constexpr int CH_NB = 64;          // Cholesky block

struct GramArgs {
  const uint16_t* x;
  const uint16_t* y;
  int64_t ldx, ldy, n_rows, rows_per_split;
  int32_t f_in, f_out, nbi, nbc, n_g, n_c, split;
  float* part;  // [batch][split][f_in][f_in + f_out]
  // problems of one launch: x, y and part of problem b at b times these
  int32_t batch;
  int64_t x_batch, y_batch;
};

// G = X^T X (tiles on and above the diagonal) and C = X^T Y over row splits,
// fp32 partial sums per split (added in fp64 afterwards).  Persistent
// workgroups of 8 waves, one per CU, take (split, tile) items; the block tile
// is 256 x 256 features, the wave tile 64 x 128 from MFMA 32x32x16 bf16.
// The K loop runs over the split's rows, 64 per step: the P part (64 rows x
// the tile's 256 row features of X) and the Q part (64 rows x its 256 column
// features of X or Y) are 32 KB each and go through a ring of five 32 KB LDS
// parts (all 160 KB), Q one step and P two steps ahead of the matrix
// instructions, filled by direct global->LDS 16-byte loads of whole 512-byte
// row pieces kept row-major; 16-byte chunks are XOR-swizzled by 4 (row mod 4)
// inside each row.  The operands want 8 consecutive rows of one feature per
// lane: the transposing LDS read of gfx950 (ds_read_b64_tr_b16) gives a lane
// 4 of them per instruction (in each group of 16 lanes, element e of lane t
// is element t mod 4 of the 8 bytes that lane 4e + t/4 addressed; so lane s
// addresses row s/4 at feature 4 (s mod 4) of a 4-row x 16-feature block and
// lane t receives rows 0..3 of feature t), and the swizzle puts the 8 rows x
// 64 bytes of one such read (two passes) in distinct banks.
__device__ __forceinline__ int gr_chunk(int r, int c) { return c ^ ((r & 3) << 2); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Rows `row`..+3 and `row`+4..+7 of feature `feat` (transposed reads by the
// lane addressing pattern above) as one 8 x bf16 operand, rows ascending.
__device__ __forceinline__ u32x4 gr_frag(const uint16_t* part, int row, int feat) {
  const char* b = reinterpret_cast<const char*>(part);
  const char* a0 = b + row * 512 + 16 * gr_chunk(row, feat >> 3) + 2 * (feat & 7);
  const char* a1 = b + (row + 4) * 512 + 16 * gr_chunk(row + 4, feat >> 3) + 2 * (feat & 7);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a1));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

struct GrItem {
  __amdgpu_buffer_rsrc_t pr, qr;  // split rows x tile features of P and Q
  uint32_t p_pitch, q_pitch;      // row pitch (bytes)
  uint32_t p_off[GR_LD], q_off[GR_LD];  // this lane's row * pitch + chunk * 16 inside a step
  int32_t nk;                     // steps of the split
  int32_t p_wrap;                 // P step k reads P rows of step k - p_wrap from step p_wrap on (k < 2 p_wrap)
};
constexpr int32_t GR_NO_WRAP = 1 << 30;

// Part of step k (64 rows) into `part`: load i of wave w covers part rows
// 2 (4w + i) and +1, lane j -> row + j/32, physical chunk j mod 32.  Steps
// past the end read nothing.
__device__ __forceinline__ void gr_issue(__amdgpu_buffer_rsrc_t r, uint32_t pitch, const uint32_t (&off)[GR_LD], int k,
                                         int nk, uint16_t* part, int32_t wrap = GR_NO_WRAP) {
  const int wave = wave_id();
  const __amdgpu_buffer_rsrc_t rr = k < nk ? r : buf_rsrc(nullptr, 0);
  const uint32_t base = static_cast<uint32_t>(k >= wrap ? k - wrap : k) * GR_BK * pitch;
#pragma unroll
  for (int i = 0; i < GR_LD; ++i) dma16(rr, base + off[i], 0, part + (wave * GR_LD + i) * 512);
}

// Load i (0..7) of a step's share of this wave: Q of step kq (loads 0..3),
// then P of step kp (4..7).  The step spreads them over its sub-steps, two
// at a time, so its products do not wait behind a burst of load issues.
__device__ __forceinline__ void gr_load(const GrItem& it, int i, int kq, int kp, uint16_t* nq, uint16_t* np) {
  const int wave = wave_id();
  if (i < GR_LD) {
    const __amdgpu_buffer_rsrc_t rr = kq < it.nk ? it.qr : buf_rsrc(nullptr, 0);
    dma16(rr, static_cast<uint32_t>(kq) * GR_BK * it.q_pitch + it.q_off[i], 0, nq + (wave * GR_LD + i) * 512);
  } else {
    const __amdgpu_buffer_rsrc_t rr = kp < it.nk ? it.pr : buf_rsrc(nullptr, 0);
    const int kw = kp >= it.p_wrap ? kp - it.p_wrap : kp;
    dma16(rr, static_cast<uint32_t>(kw) * GR_BK * it.p_pitch + it.p_off[i - GR_LD], 0,
          np + (wave * GR_LD + i - GR_LD) * 512);
  }
}

// One step: 4 x (2 P + 4 Q fragments, 8 MFMAs); with ISSUE, the loads of Q
// of step kq and P of step kp are issued two per sub-step.
template <bool ISSUE = false>
__device__ __forceinline__ void gr_compute(const uint16_t* pp, const uint16_t* pq, f32x16 (&acc)[2][4],
                                           const GrItem* it = nullptr, int kq = 0, int kp = 0,
                                           uint16_t* nq = nullptr, uint16_t* np = nullptr) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;
  // lane of a 16-lane group g: the MFMA operand of lane l covers features
  // l mod 32 and rows 8 (l / 32) .. +7
  const int g = lane >> 4, s = lane & 15;
  const int r0 = 8 * (g >> 1) + (s >> 2);
  const int f0 = 16 * (g & 1) + 4 * (s & 3);
#pragma unroll
  for (int kk = 0; kk < GR_BK / 16; ++kk) {
    if constexpr (ISSUE) {
      __builtin_amdgcn_sched_barrier(0);
      gr_load(*it, 2 * kk, kq, kp, nq, np);
      gr_load(*it, 2 * kk + 1, kq, kp, nq, np);
      __builtin_amdgcn_sched_barrier(0);
    }
    u32x4 af[2], bf[4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) af[mi] = gr_frag(pp, 16 * kk + r0, wm * 64 + mi * 32 + f0);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) bf[ni] = gr_frag(pq, 16 * kk + r0, wn * 128 + ni * 32 + f0);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[mi]),
                                                              __builtin_bit_cast(bf16x8, bf[ni]), acc[mi][ni], 0, 0, 0);
  }
}

__device__ __forceinline__ void gr_sync() {
  KVX_WAIT_VM(GR_LD);
  KVX_COMPILER_FENCE();
  __builtin_amdgcn_s_barrier();
  KVX_COMPILER_FENCE();
}

// P of step k in part 2k mod 5, Q in part 2k+1 mod 5; the step issues Q of
// k+1 and P of k+2 into the two parts of step k-1.
#define GR_STEP(K, PA, PB, NB, NA, LIVE)                   \
  gr_sync();                                               \
  gr_issue(it.qr, it.q_pitch, it.q_off, (K) + 1, it.nk, NB); \
  gr_issue(it.pr, it.p_pitch, it.p_off, (K) + 2, it.nk, NA, it.p_wrap); \
  if (LIVE) gr_compute(PA, PB, acc);
// A whole step (no tail): loads spread over the sub-steps.
#define GR_STEP_FULL(K, PA, PB, NB, NA)                    \
  gr_sync();                                               \
  gr_compute<true>(PA, PB, acc, &it, (K) + 1, (K) + 2, NB, NA);

__global__ __attribute__((amdgpu_flat_work_group_size(GR_THREADS, GR_THREADS), amdgpu_waves_per_eu(2, 2))) void
gram_kernel(const GramArgs g) {
  __shared__ __attribute__((aligned(1024))) uint16_t p0[GR_PART];
  __shared__ __attribute__((aligned(1024))) uint16_t p1[GR_PART];
  __shared__ __attribute__((aligned(1024))) uint16_t p2[GR_PART];
  __shared__ __attribute__((aligned(1024))) uint16_t p3[GR_PART];
  __shared__ __attribute__((aligned(1024))) uint16_t p4[GR_PART];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;
  const int32_t per = g.n_g + g.n_c;
  const int64_t per_prob = static_cast<int64_t>(g.split) * per;
  const int64_t T = g.batch * per_prob;
  const int32_t G = gridDim.x;
  // consecutive items go to the workgroups of one XCD (dispatch is round
  // robin over the 8 XCDs)
  const int32_t slot = (G % 8 == 0) ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int64_t ldp = static_cast<int64_t>(g.f_in) + g.f_out;

  for (int64_t t = slot; t < T; t += G) {
    const int64_t prob = t / per_prob;
    const int32_t sidx = static_cast<int32_t>((t % per_prob) / per);
    int32_t tt = static_cast<int32_t>((t % per_prob) % per);
    const uint16_t* gx = g.x + prob * g.x_batch;
    const uint16_t* gy = g.y + prob * g.y_batch;
    int32_t bi, bj;
    bool is_c;
    if (tt < g.n_g) {  // upper-triangle tile index -> (bi, bj), bi <= bj
      is_c = false;
      bi = 0;
      int32_t rowlen = g.nbi;
      while (tt >= rowlen) {
        tt -= rowlen;
        ++bi;
        --rowlen;
      }
      bj = bi + tt;
    } else {
      is_c = true;
      tt -= g.n_g;
      bi = tt / g.nbc;
      bj = tt % g.nbc;
    }
    const int64_t k_begin = static_cast<int64_t>(sidx) * g.rows_per_split;
    int64_t rows = g.n_rows - k_begin;
    if (rows > g.rows_per_split) rows = g.rows_per_split;
    if (rows < 0) rows = 0;
    const int32_t i0 = bi * GR_T, j0 = bj * GR_T;
    const uint16_t* q = is_c ? gy : gx;
    const int64_t ldq = is_c ? g.ldy : g.ldx;
    const int32_t fq = is_c ? g.f_out : g.f_in;

    GrItem it;
    it.p_pitch = static_cast<uint32_t>(2 * g.ldx);
    it.q_pitch = static_cast<uint32_t>(2 * ldq);
    // the range ends with the split's last row (features past the row's end
    // come from the next row and only reach outputs that are not written)
    it.pr = buf_rsrc(gx + k_begin * g.ldx + i0, static_cast<uint32_t>(rows * 2 * g.ldx - 2 * i0));
    it.qr = buf_rsrc(q + k_begin * ldq + j0, static_cast<uint32_t>(rows * 2 * ldq - 2 * j0));
    if (rows == 0) {
      it.pr = buf_rsrc(nullptr, 0);
      it.qr = buf_rsrc(nullptr, 0);
    }
    it.nk = static_cast<int32_t>((rows + GR_BK - 1) / GR_BK);
    it.p_wrap = GR_NO_WRAP;
#pragma unroll
    for (int i = 0; i < GR_LD; ++i) {
      const int row = 2 * (wave * GR_LD + i) + (lane >> 5);
      const int pc = gr_chunk(row, lane & 31);  // logical chunk of physical position lane % 32
      it.p_off[i] = static_cast<uint32_t>(row) * it.p_pitch + 16u * pc;
      it.q_off[i] = static_cast<uint32_t>(row) * it.q_pitch + 16u * pc;
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (it.nk > 0) {
      gr_issue(it.pr, it.p_pitch, it.p_off, 0, it.nk, p0);
      gr_issue(it.qr, it.q_pitch, it.q_off, 0, it.nk, p1);
      gr_issue(it.pr, it.p_pitch, it.p_off, 1, it.nk, p2);
      // whole groups of five steps without branches, then the 1..4
      // remaining steps (a per-step branch would make the compiler drain
      // every load before the first fragment read of a step)
      int k = 0;
      for (; k + 5 <= it.nk; k += 5) {
        GR_STEP_FULL(k, p0, p1, p3, p4)
        GR_STEP_FULL(k + 1, p2, p3, p0, p1)
        GR_STEP_FULL(k + 2, p4, p0, p2, p3)
        GR_STEP_FULL(k + 3, p1, p2, p4, p0)
        GR_STEP_FULL(k + 4, p3, p4, p1, p2)
      }
      if (k < it.nk) {
        GR_STEP(k, p0, p1, p3, p4, true)
        GR_STEP(k + 1, p2, p3, p0, p1, k + 1 < it.nk)
        GR_STEP(k + 2, p4, p0, p2, p3, k + 2 < it.nk)
        GR_STEP(k + 3, p1, p2, p4, p0, k + 3 < it.nk)
        GR_STEP(k + 4, p3, p4, p1, p2, k + 4 < it.nk)
      }
      KVX_WAIT_VM(0);
    }

    float* part = g.part + (prob * g.split + sidx) * g.f_in * ldp + (is_c ? g.f_in : 0);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t i = i0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int32_t j = j0 + wn * 128 + ni * 32 + (lane & 31);
          if (i < g.f_in && j < fq) part[static_cast<int64_t>(i) * ldp + j] = acc[mi][ni][r];
        }
    // every wave is past its last step before the next item's loads land
    __syncthreads();
  }
}

// ---------------------------------------------------------------- Gram from runs of the alignment
//
// The features of a calibration row are the sender rows of its aligned
// sender token, so within a run u of receiver tokens that share one sender
// token (length c_u) every feature row is the same row x_u.  Then
//   X^T X = sum_u c_u x_u x_u^T = sum_j 2^j sum_{u : bit j of c_u} x_u x_u^T
// (runs of 2^15 or more tokens add their c_u >> 15 to group 15), and with the
// groups taken from the largest j down, each group's sum accumulated on top
// of the accumulator doubled 2^(j_prev - j) times (exact) leaves
// sum_j 2^j G_j after the last group and a final scaling by 2^(j_last).  The
// products are the exact bf16 products of the plain Gram, summed in fp32.
// X^T Y = sum_u x_u s_u^T with s_u the run's target sum, taken as a high and
// a low bf16 part: the distinct rows x_u are read twice, once against the
// high parts and once against the low parts.
// A launch covers every problem (receiver layer) of one role, with the full
// row range per item, so no split partials are kept.  Items are the distinct
// lower tiles of G over all problems (receiver layers whose taps pair the
// same sender layers at the same offsets share a tile: formed once, written
// to each) and the (problem, tile) items of C.  G is written on and below
// the diagonal tiles only: the Cholesky factorisation, the solves and the
// trace read nothing else.
constexpr int GRR_BLOCK = 5;                    // steps per unrolled block of the K loop
constexpr int GRR_PAD = GRR_BLOCK * GR_BK;      // rows of each bit group padded to whole blocks
constexpr int GRR_MAX_GROUPS = 16;

// One distinct lower tile of G: sender layer and row offset of its row side
// (a) and column side (b), and its consumers dests[first .. first + count).
// Receiver layers whose taps pair the same sender layers at the same offsets
// share the tile: it is formed once and written to each of them.
struct GrrKey {
  int32_t la, oa, lb, ob, first, count, pad0, pad1;
};
// A consumer: problem, tile position (bi, bj) in its G, and whether it takes
// the tile transposed (its row side is the key's b side).
struct GrrDest {
  int32_t prob, bi, bj, trans;
};
typedef const __attribute__((address_space(4))) GrrKey* grr_key_ptr;
typedef const __attribute__((address_space(4))) GrrDest* grr_dest_ptr;

struct GramRunsArgs {
  const uint16_t* xg;       // [L_S][xg_rows][row]: the bit-group rows of every sender layer
  const uint16_t* xu;       // [L_S][u_pad][row]: the distinct rows x_u
  const uint16_t* qp;       // [problems][2 u_pad][f_out]: run sums of the targets, high then low parts
  int64_t xg_layer, xu_layer, qp_layer;  // element strides between layers (problems for qp)
  const int32_t* taps;      // device [problems][n_taps]: sender layer of each tap
  double* G;                // problem p's G (f_in x f_in) and C (f_in x f_out) at p * bs
  double* C;
  int64_t bs;
  const GrrKey* keys;       // [n_keys] distinct G tiles (read as uniform scalar loads)
  const GrrDest* dests;     // their consumers
  int32_t n_keys;
  int32_t row, xg_rows, u_pad, n_taps, n_problems;
  int32_t f_in, f_out, nbi, nbc, n_g, n_c;
  int32_t n_groups;
  int32_t grp_end[GRR_MAX_GROUPS];  // block (of GRR_BLOCK steps) after which group g ends
  int32_t grp_exp[GRR_MAX_GROUPS];  // its bit j
};

// arr[idx] of a kernel-argument array with constant indices only (stays in
// scalar registers, no memory access inside the K loop)
__device__ __forceinline__ int32_t grr_pick(const int32_t (&arr)[GRR_MAX_GROUPS], int32_t idx) {
  int32_t v = 0;
#pragma unroll
  for (int i = 0; i < GRR_MAX_GROUPS; ++i) v = (i == idx) ? arr[i] : v;
  return v;
}

__global__ __attribute__((amdgpu_flat_work_group_size(GR_THREADS, GR_THREADS), amdgpu_waves_per_eu(2, 2))) void
gram_runs_kernel(const GramRunsArgs g) {
  __shared__ __attribute__((aligned(1024))) uint16_t p0[GR_PART];
  __shared__ __attribute__((aligned(1024))) uint16_t p1[GR_PART];
  __shared__ __attribute__((aligned(1024))) uint16_t p2[GR_PART];
  __shared__ __attribute__((aligned(1024))) uint16_t p3[GR_PART];
  __shared__ __attribute__((aligned(1024))) uint16_t p4[GR_PART];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;
  // items: the distinct G tiles, then (problem, C tile)
  const int64_t T = g.n_keys + static_cast<int64_t>(g.n_problems) * g.n_c;
  const int32_t NG = gridDim.x;
  const int32_t slot = (NG % 8 == 0) ? (blockIdx.x & 7) * (NG >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const uint32_t xpitch = static_cast<uint32_t>(2 * g.row);
  const grr_key_ptr keys = (grr_key_ptr)(g.keys);  // constant address space: scalar loads
  const grr_dest_ptr dests = (grr_dest_ptr)(g.dests);

  for (int64_t t = slot; t < T; t += NG) {
    const bool is_c = t >= g.n_keys;
    int32_t prob = 0, bi = 0, bj = 0, tap_i, off_i, key = 0;
    if (is_c) {
      const int32_t tt = static_cast<int32_t>(t - g.n_keys);
      prob = tt / g.n_c;
      bi = (tt % g.n_c) / g.nbc;
      bj = (tt % g.n_c) % g.nbc;
      // feature tile bi lies inside one tap's row (row is a multiple of 256)
      tap_i = g.taps[static_cast<int64_t>(prob) * g.n_taps + bi * GR_T / g.row];
      off_i = bi * GR_T % g.row;
    } else {
      key = static_cast<int32_t>(t);
      tap_i = keys[key].la;
      off_i = keys[key].oa;
    }
    const int32_t j0 = bj * GR_T;

    GrItem it;
    it.p_pitch = xpitch;
    if (is_c) {
      const uint16_t* pb = g.xu + tap_i * g.xu_layer + off_i;
      const uint16_t* qb = g.qp + prob * g.qp_layer + j0;
      it.pr = buf_rsrc(pb, static_cast<uint32_t>(static_cast<int64_t>(g.u_pad) * xpitch - 2 * off_i));
      it.q_pitch = static_cast<uint32_t>(2 * g.f_out);
      it.qr = buf_rsrc(qb, static_cast<uint32_t>(2LL * g.u_pad * it.q_pitch - 2 * j0));
      it.p_wrap = g.u_pad / GR_BK;
      it.nk = 2 * it.p_wrap;
    } else {
      const int32_t tap_j = keys[key].lb;
      const int32_t off_j = keys[key].ob;
      const uint16_t* pb = g.xg + tap_i * g.xg_layer + off_i;
      const uint16_t* qb = g.xg + tap_j * g.xg_layer + off_j;
      it.pr = buf_rsrc(pb, static_cast<uint32_t>(static_cast<int64_t>(g.xg_rows) * xpitch - 2 * off_i));
      it.q_pitch = xpitch;
      it.qr = buf_rsrc(qb, static_cast<uint32_t>(static_cast<int64_t>(g.xg_rows) * xpitch - 2 * off_j));
      it.p_wrap = GR_NO_WRAP;
      it.nk = g.xg_rows / GR_BK;  // whole blocks: each bit group ends on a block boundary
    }
    if (it.nk == 0) {
      it.pr = buf_rsrc(nullptr, 0);
      it.qr = buf_rsrc(nullptr, 0);
    }
#pragma unroll
    for (int i = 0; i < GR_LD; ++i) {
      const int r = 2 * (wave * GR_LD + i) + (lane >> 5);
      const int pc = gr_chunk(r, lane & 31);
      it.p_off[i] = static_cast<uint32_t>(r) * it.p_pitch + 16u * pc;
      it.q_off[i] = static_cast<uint32_t>(r) * it.q_pitch + 16u * pc;
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (it.nk > 0) {
      gr_issue(it.pr, it.p_pitch, it.p_off, 0, it.nk, p0, it.p_wrap);
      gr_issue(it.qr, it.q_pitch, it.q_off, 0, it.nk, p1);
      gr_issue(it.pr, it.p_pitch, it.p_off, 1, it.nk, p2, it.p_wrap);
      int32_t grp = 0;                                   // current bit group (G items)
      int32_t grp_end = is_c ? -1 : grr_pick(g.grp_end, 0);
      int k = 0;
      for (; k + GRR_BLOCK <= it.nk; k += GRR_BLOCK) {
        GR_STEP_FULL(k, p0, p1, p3, p4)
        GR_STEP_FULL(k + 1, p2, p3, p0, p1)
        GR_STEP_FULL(k + 2, p4, p0, p2, p3)
        GR_STEP_FULL(k + 3, p1, p2, p4, p0)
        GR_STEP_FULL(k + 4, p3, p4, p1, p2)
        if ((k + GRR_BLOCK) / GRR_BLOCK == grp_end) {
          // end of bit group grp: double the sums (j_grp - j_next) times,
          // j_next = 0 after the last group
          const int32_t e_now = grr_pick(g.grp_exp, grp);
          const int32_t e_next = grp + 1 < g.n_groups ? grr_pick(g.grp_exp, grp + 1) : 0;
          const float f = __uint_as_float(static_cast<uint32_t>(127 + e_now - e_next) << 23);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int e = 0; e < 16; ++e) acc[i][j][e] *= f;
          ++grp;
          grp_end = grp < g.n_groups ? grr_pick(g.grp_end, grp) : -1;
        }
      }
      if (k < it.nk) {  // C items only: the 1..4 remaining steps
        GR_STEP(k, p0, p1, p3, p4, true)
        GR_STEP(k + 1, p2, p3, p0, p1, k + 1 < it.nk)
        GR_STEP(k + 2, p4, p0, p2, p3, k + 2 < it.nk)
        GR_STEP(k + 3, p1, p2, p4, p0, k + 3 < it.nk)
        GR_STEP(k + 4, p3, p4, p1, p2, k + 4 < it.nk)
      }
      KVX_WAIT_VM(0);
    }

    // tile-local row (P side) and column (Q side) of accumulator element
    // (mi, ni, r) of this lane
    auto lrow = [&](int mi, int r) { return wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); };
    auto lcol = [&](int ni) { return wn * 128 + ni * 32 + (lane & 31); };
    if (is_c) {
      double* C = g.C + prob * g.bs;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int32_t i = bi * GR_T + lrow(mi, r), j = j0 + lcol(ni);
            if (i < g.f_in && j < g.f_out) C[static_cast<int64_t>(i) * g.f_out + j] = static_cast<double>(acc[mi][ni][r]);
          }
    } else {
      const int32_t first = keys[key].first, count = keys[key].count;
      for (int32_t d = 0; d < count; ++d) {
        const int32_t dp = dests[first + d].prob, dbi = dests[first + d].bi, dbj = dests[first + d].bj;
        const bool tr = dests[first + d].trans != 0;
        double* G = g.G + dp * g.bs;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              // not transposed: the tile's rows are the consumer's rows
              const int32_t i = dbi * GR_T + (tr ? lcol(ni) : lrow(mi, r));
              const int32_t j = dbj * GR_T + (tr ? lrow(mi, r) : lcol(ni));
              // converted per store: hoisted out of the consumer loop, the
              // 128 fp64 values would not fit the registers
              float a = acc[mi][ni][r];
              asm volatile("" : "+v"(a));
              G[static_cast<int64_t>(i) * g.f_in + j] = static_cast<double>(a);
            }
      }
    }
    __syncthreads();
  }
}

// One 16-byte piece of a row, or with ROT (keys stored rotated) the pieces
// of 8 pairs (c .. c+7 and c+d/2 .. c+d/2+7 of a head of d) rotated back
// at the row's position (its token index) from the fp32 (cos, sin) table,
// rounded to bf16.  Row r takes token uniq[u] of u = list[r] (or u = r below
// n_valid, zero past it); without uniq the token is u itself.
template <bool ROT>
__global__ __launch_bounds__(256) void fitc_gather_kernel(const uint16_t* __restrict__ send, int64_t send_layer,
                                                          int32_t row, const int32_t* __restrict__ uniq,
                                                          const int32_t* __restrict__ list, int32_t n_valid,
                                                          int32_t rows_out, uint16_t* __restrict__ out,
                                                          int64_t out_layer, const float2* __restrict__ tab,
                                                          int32_t hd) {
  const int64_t sl = blockIdx.y;
  const int32_t cpr = ROT ? row / 16 : row / 8;
  const int64_t total = static_cast<int64_t>(rows_out) * cpr;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; t < total;
       t += static_cast<int64_t>(gridDim.x) * 256) {
    const int32_t r = static_cast<int32_t>(t / cpr), c = static_cast<int32_t>(t % cpr);
    const int32_t u = list ? list[r] : (r < n_valid ? r : -1);
    const int64_t tok = u < 0 ? 0 : (uniq ? uniq[u] : u);
    const uint16_t* src = send + sl * send_layer + tok * row;
    uint16_t* dst = out + sl * out_layer + static_cast<int64_t>(r) * row;
    if constexpr (!ROT) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (u >= 0) v = *reinterpret_cast<const u32x4*>(src + 8 * c);
      *reinterpret_cast<u32x4*>(dst + 8 * c) = v;
    } else {
      const int32_t qh = hd / 16;  // pieces per half head
      const int32_t ca = (c / qh) * hd + 8 * (c % qh), cb = ca + hd / 2;
      u32x4 va = u32x4{0u, 0u, 0u, 0u}, vb = va;
      if (u >= 0) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(src + ca);
        const u32x4 b = *reinterpret_cast<const u32x4*>(src + cb);
        const float2* cs = tab + tok * (hd / 2) + 8 * (c % qh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 c0 = cs[2 * e], c1 = cs[2 * e + 1];
          const float a0 = bf16lo(a[e]), a1 = bf16hi(a[e]), b0 = bf16lo(b[e]), b1 = bf16hi(b[e]);
          // rotation by -angle: (a, b) -> (a cos + b sin, b cos - a sin)
          va[e] = pack_bf16(a0 * c0.x + b0 * c0.y, a1 * c1.x + b1 * c1.y);
          vb[e] = pack_bf16(b0 * c0.x - a0 * c0.y, b1 * c1.x - a1 * c1.y);
        }
      }
      *reinterpret_cast<u32x4*>(dst + ca) = va;
      *reinterpret_cast<u32x4*>(dst + cb) = vb;
    }
  }
}

// Run sums of the targets: for run u of every receiver layer, the sum over its
// receiver rows in token order, fp32, stored as a high bf16 part (rows
// 0 .. u_pad) and the bf16 rounding of the remainder (rows u_pad .. 2 u_pad);
// padding runs get zeros.  One thread: one 16-byte piece, or with ROT (target
// keys stored rotated) the two pieces of 8 pairs, each row rotated back at
// its position (its token index) before it is added.
template <bool ROT>
__global__ __launch_bounds__(256) void fitc_target_sums_kernel(const uint16_t* __restrict__ y, int64_t y_layer,
                                                               int32_t f_out, const int32_t* __restrict__ run_begin,
                                                               int32_t n_runs, int32_t u_pad,
                                                               uint16_t* __restrict__ qp, int64_t qp_layer,
                                                               const float2* __restrict__ tab, int32_t hd) {
  constexpr int NP = ROT ? 2 : 1;  // pieces per thread
  const int64_t l = blockIdx.y;
  const int32_t cpr = f_out / (8 * NP);
  const int64_t total = static_cast<int64_t>(u_pad) * cpr;
  const uint16_t* yl = y + l * y_layer;
  uint16_t* ql = qp + l * qp_layer;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; t < total;
       t += static_cast<int64_t>(gridDim.x) * 256) {
    const int32_t u = static_cast<int32_t>(t / cpr), c = static_cast<int32_t>(t % cpr);
    int32_t col[NP];
    if constexpr (ROT) {
      const int32_t qh = hd / 16;
      col[0] = (c / qh) * hd + 8 * (c % qh);
      col[NP - 1] = col[0] + hd / 2;
    } else {
      col[0] = 8 * c;
    }
    float sum[NP][8];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[p][e] = 0.0f;
    if (u < n_runs) {
      for (int32_t i = run_begin[u]; i < run_begin[u + 1]; ++i) {
        const uint16_t* yr = yl + static_cast<int64_t>(i) * f_out;
        if constexpr (ROT) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(yr + col[0]);
          const u32x4 b = *reinterpret_cast<const u32x4*>(yr + col[NP - 1]);
          const float2* cs = tab + static_cast<int64_t>(i) * (hd / 2) + 8 * (c % (hd / 16));
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float2 q = cs[e];
            const float av = (e & 1) ? bf16hi(a[e >> 1]) : bf16lo(a[e >> 1]);
            const float bv = (e & 1) ? bf16hi(b[e >> 1]) : bf16lo(b[e >> 1]);
            sum[0][e] += av * q.x + bv * q.y;
            sum[NP - 1][e] += bv * q.x - av * q.y;
          }
        } else {
          const u32x4 v = *reinterpret_cast<const u32x4*>(yr + col[0]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sum[0][2 * e] += bf16lo(v[e]);
            sum[0][2 * e + 1] += bf16hi(v[e]);
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      u32x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t h0 = f32_to_bf16_rne(sum[p][2 * e]), h1 = f32_to_bf16_rne(sum[p][2 * e + 1]);
        const uint16_t l0 = f32_to_bf16_rne(sum[p][2 * e] - bf16_to_f32(h0));
        const uint16_t l1 = f32_to_bf16_rne(sum[p][2 * e + 1] - bf16_to_f32(h1));
        hi[e] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
        lo[e] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
      }
      *reinterpret_cast<u32x4*>(ql + static_cast<int64_t>(u) * f_out + col[p]) = hi;
      *reinterpret_cast<u32x4*>(ql + (static_cast<int64_t>(u_pad) + u) * f_out + col[p]) = lo;
    }
  }
}

#undef GR_STEP
#undef GR_STEP_FULL

// fp32 inputs: G, C and column sums in fp64 by plain loops (small fits).
__global__ __launch_bounds__(256) void gram_f32_kernel(const float* __restrict__ x, int64_t ldx,
                                                       const float* __restrict__ y, int64_t ldy,
                                                       int64_t n_rows, int32_t f_in, int32_t f_out,
                                                       double* __restrict__ G, double* __restrict__ C) {
  const int64_t total = static_cast<int64_t>(f_in) * (f_in + f_out);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int32_t i = static_cast<int32_t>(e / (f_in + f_out));
    const int32_t j = static_cast<int32_t>(e % (f_in + f_out));
    double s = 0.0;
    if (j < f_in) {
      for (int64_t k = 0; k < n_rows; ++k) s += static_cast<double>(x[k * ldx + i]) * x[k * ldx + j];
      G[static_cast<int64_t>(i) * f_in + j] = s;
    } else {
      const int32_t jj = j - f_in;
      for (int64_t k = 0; k < n_rows; ++k) s += static_cast<double>(x[k * ldx + i]) * y[k * ldy + jj];
      C[static_cast<int64_t>(i) * f_out + jj] = s;
    }
  }
}

// Column sums of X and Y in fp64 (for the intercept and the moments), in
// two passes with a fixed summation order: workgroup (g, r) adds rows
// r * rows_per_chunk .. of its 256 V columns (V = 8 bf16 columns per 16-byte
// load, or 1 fp32 column) into partial[r][col]; then each column's
// CS_CHUNKS partials are added in chunk order.  bf16 callers guarantee
// cols % 8 == 0, ld % 8 == 0 and a 16-byte aligned base.
constexpr int CS_CHUNKS = 512;
template <bool F32>
__global__ __launch_bounds__(256) void colsum_part_kernel(const void* __restrict__ m, int64_t ld, int64_t n_rows,
                                                          int32_t cols, int64_t rows_per_chunk,
                                                          double* __restrict__ partial, int64_t m_batch) {
  // problem blockIdx.z: its rows m_batch elements after the previous
  // problem's, its partials gridDim.y chunks after them
  constexpr int V = F32 ? 1 : 8;
  const int32_t c0 = (blockIdx.x * 256 + threadIdx.x) * V;
  if (c0 >= cols) return;
  if constexpr (F32)
    m = static_cast<const float*>(m) + blockIdx.z * m_batch;
  else
    m = static_cast<const uint16_t*>(m) + blockIdx.z * m_batch;
  partial += static_cast<int64_t>(blockIdx.z) * gridDim.y * cols;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * rows_per_chunk;
  const int64_t r1 = min(n_rows, r0 + rows_per_chunk);
  double acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0;
  for (int64_t r = r0; r < r1; ++r) {
    if constexpr (F32) {
      acc[0] += static_cast<double>(static_cast<const float*>(m)[r * ld + c0]);
    } else {
      const u32x4 q = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(m) + r * ld + c0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += static_cast<double>(bf16lo(q[e]));
        acc[2 * e + 1] += static_cast<double>(bf16hi(q[e]));
      }
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) partial[static_cast<int64_t>(blockIdx.y) * cols + c0 + v] = acc[v];
}

__global__ __launch_bounds__(256) void colsum_reduce_kernel(const double* __restrict__ partial, int32_t cols,
                                                            int32_t chunks, double* __restrict__ out,
                                                            int64_t out_batch) {
  // problem blockIdx.y: chunks partials of cols each, added in chunk order
  const int32_t c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  partial += static_cast<int64_t>(blockIdx.y) * chunks * cols;
  double s = 0.0;
  for (int q = 0; q < chunks; ++q) s += partial[static_cast<int64_t>(q) * cols + c];
  out[static_cast<int64_t>(blockIdx.y) * out_batch + c] = s;
}

static int colsum(const void* m, int64_t ld, int64_t n_rows, int32_t cols, int32_t f32, double* partial, double* out,
                  hipStream_t s) {
  const int64_t rpc = (n_rows + CS_CHUNKS - 1) / CS_CHUNKS;
  const int v = f32 ? 1 : 8;
  const dim3 grid(static_cast<unsigned>(ceil_div(cols, 256 * v)), CS_CHUNKS);
  if (f32)
    colsum_part_kernel<true><<<grid, 256, 0, s>>>(m, ld, n_rows, cols, rpc, partial, 0);
  else
    colsum_part_kernel<false><<<grid, 256, 0, s>>>(m, ld, n_rows, cols, rpc, partial, 0);
  colsum_reduce_kernel<<<static_cast<unsigned>(ceil_div(cols, 256)), 256, 0, s>>>(partial, cols, CS_CHUNKS, out, 0);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// Column sums of `batch` bf16 matrices of one shape in one pass: problem b's
// rows m_batch elements after problem a's, its sums at out + b out_batch;
// `partial` has room for cap doubles (as many row chunks as fit, at most
// CS_CHUNKS; one problem at a time when not even one chunk per problem fits).
static int colsum_batch(const uint16_t* m, int64_t ld, int64_t m_batch, int64_t n_rows, int32_t cols, int32_t batch,
                        double* partial, int64_t cap, double* out, int64_t out_batch, hipStream_t s) {
  const int64_t chunks = std::min<int64_t>(CS_CHUNKS, cap / (static_cast<int64_t>(cols) * batch));
  if (chunks < 1) {
    for (int32_t b = 0; b < batch; ++b)
      if (int st = colsum(m + b * m_batch, ld, n_rows, cols, 0, partial, out + b * out_batch, s)) return st;
    return KVX_OK;
  }
  const int64_t rpc = ceil_div(n_rows, chunks);
  const dim3 grid(static_cast<unsigned>(ceil_div(cols, 256 * 8)), static_cast<unsigned>(chunks),
                  static_cast<unsigned>(batch));
  colsum_part_kernel<false><<<grid, 256, 0, s>>>(m, ld, n_rows, cols, rpc, partial, m_batch);
  colsum_reduce_kernel<<<dim3(static_cast<unsigned>(ceil_div(cols, 256)), static_cast<unsigned>(batch)), 256, 0,
                         s>>>(partial, cols, static_cast<int32_t>(chunks), out, out_batch);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// Sum of the split partials in fp64 by 64 x 64 blocks of [G | C]: blocks of
// G on and above the diagonal and every block of C are read row by row
// (256-byte rows of each split); a block of G above the diagonal is also
// written to its mirror through an LDS transpose, so every global access
// walks rows.
constexpr int RD_T = 64;
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ part, int32_t split,
                                                          int32_t f_in, int32_t f_out, double* __restrict__ G,
                                                          double* __restrict__ C, int64_t bs) {
  __shared__ double tr[RD_T][RD_T + 1];
  // problem blockIdx.y: its split partials follow the previous problem's,
  // its G and C sit bs doubles after the previous problem's
  part += static_cast<int64_t>(blockIdx.y) * split * f_in * (static_cast<int64_t>(f_in) + f_out);
  G += static_cast<int64_t>(blockIdx.y) * bs;
  if (C) C += static_cast<int64_t>(blockIdx.y) * bs;
  const int32_t nbi = (f_in + RD_T - 1) / RD_T;
  const int32_t nbc = (f_out + RD_T - 1) / RD_T;
  const int32_t n_g = nbi * (nbi + 1) / 2;
  int32_t t = blockIdx.x;
  int32_t bi, bj;
  bool is_c;
  if (t < n_g) {
    is_c = false;
    bi = 0;
    int32_t rowlen = nbi;
    while (t >= rowlen) {
      t -= rowlen;
      ++bi;
      --rowlen;
    }
    bj = bi + t;
  } else {
    is_c = true;
    t -= n_g;
    bi = t / nbc;
    bj = t % nbc;
  }
  const int64_t ldp = static_cast<int64_t>(f_in) + f_out;
  const int64_t total = static_cast<int64_t>(f_in) * ldp;
  const int32_t fq = is_c ? f_out : f_in;
  const int c = threadIdx.x & 63, r4 = threadIdx.x >> 6;
  const int32_t j = bj * RD_T + c;
#pragma unroll 4
  for (int rr = 0; rr < RD_T; rr += 4) {
    const int32_t i = bi * RD_T + rr + r4;
    if (i < f_in && j < fq) {
      const int64_t src = static_cast<int64_t>(i) * ldp + (is_c ? f_in : 0) + j;
      double v = 0.0;
      for (int32_t q = 0; q < split; ++q) v += static_cast<double>(part[static_cast<int64_t>(q) * total + src]);
      if (is_c)
        C[static_cast<int64_t>(i) * f_out + j] = v;
      else
        G[static_cast<int64_t>(i) * f_in + j] = v;
      tr[rr + r4][c] = v;
    }
  }
  if (is_c || bi == bj) return;
  __syncthreads();
  // mirror: G[j][i] for the block's columns j as rows
#pragma unroll 4
  for (int rr = 0; rr < RD_T; rr += 4) {
    const int32_t jj = bj * RD_T + rr + r4;  // row of the mirror
    const int32_t ii = bi * RD_T + c;        // column of the mirror
    if (jj < f_in && ii < f_in) G[static_cast<int64_t>(jj) * f_in + ii] = tr[c][rr + r4];
  }
}

// Centring: G -= sx sx^T / n, C -= sx sy^T / n; problem blockIdx.y has its
// G, C, sx and sy bs doubles after the previous problem's.
__global__ __launch_bounds__(256) void center_kernel(double* __restrict__ G, double* __restrict__ C,
                                                     const double* __restrict__ sx, const double* __restrict__ sy,
                                                     int32_t f_in, int32_t f_out, double inv_n, int64_t bs) {
  const int64_t z = static_cast<int64_t>(blockIdx.y) * bs;
  G += z;
  sx += z;
  sy += z;
  if (C) C += z;
  const int64_t ld = static_cast<int64_t>(f_in) + f_out;
  const int64_t total = static_cast<int64_t>(f_in) * ld;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int32_t i = static_cast<int32_t>(e / ld);
    const int32_t j = static_cast<int32_t>(e % ld);
    if (j < f_in) G[static_cast<int64_t>(i) * f_in + j] -= sx[i] * sx[j] * inv_n;
    else C[static_cast<int64_t>(i) * f_out + (j - f_in)] -= sx[i] * sy[j - f_in] * inv_n;
  }
}

// lambda = abs + rel * trace(G) / f_in, added to the diagonal (one block,
// fixed summation order).
__global__ __launch_bounds__(256) void lambda_kernel(double* __restrict__ G, int32_t f_in, double lam_abs,
                                                     double lam_rel, double* __restrict__ lam_out) {
  __shared__ double red[256];
  double s = 0.0;
  for (int32_t i = threadIdx.x; i < f_in; i += 256) s += G[static_cast<int64_t>(i) * f_in + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double lam = lam_abs + lam_rel * red[0] / static_cast<double>(f_in);
  for (int32_t i = threadIdx.x; i < f_in; i += 256) G[static_cast<int64_t>(i) * f_in + i] += lam;
  if (threadIdx.x == 0) *lam_out = lam;
}

// ---------------------------------------------------------------- fp64 Cholesky pieces

// A double of lane l (l uniform), as two 32-bit lane reads.
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(v));
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(u & 0xffffffffu), l));
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), l));
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

// Factor the diagonal block [k0, k0+nb) (lower) of one problem of a batch
// (one workgroup per problem), flag non-positive pivots,
// and write the inverse of the factor (lower, nb x nb, zero above the
// diagonal, row stride CH_NB) to `linv`: the panel and the block triangular
// solves then become products with it.  One wave.  The block's lower
// triangle is read a row at a time (lane = column, whole rows per load) and
// turned through LDS so that lane i holds row i in registers.  At column j
// every lane publishes its entry of the column in LDS and reads the whole
// column back, two entries per read that every lane shares (one wave: its
// LDS operations execute in order); the square root and its reciprocal are
// recomputed per lane, each lane scales its own entry and updates the rest
// of its row with the column scaled by the reciprocal (folded into the
// lane's multiplier).  Entries above the diagonal take updates too and are
// never read.  Rows past nb are the identity.  The factor goes back through
// LDS (lane = column on the way out), and the inverse is formed one column
// per lane by forward substitution against it, each factor entry one LDS
// read that every lane shares, the division by the pivot a product with the
// reciprocal held by the pivot's lane.
__global__ __launch_bounds__(64) void potrf_diag_kernel(double* __restrict__ A, int64_t bsa, int32_t n, int32_t k0,
                                                        int32_t nb, int32_t* __restrict__ flag,
                                                        double* __restrict__ linv, int64_t bsl) {
  // problem blockIdx.x of a batch
  A += blockIdx.x * bsa;
  flag += blockIdx.x;
  linv += blockIdx.x * bsl;
  __shared__ double L[CH_NB][CH_NB + 1];
  __shared__ __align__(16) double col[CH_NB];
  const int i = threadIdx.x;
  {
    // every row's load in flight at once (the block was just updated, often by another XCD)
    double in[CH_NB];
#pragma unroll
    for (int r = 0; r < CH_NB; ++r)
      in[r] = (r < nb && i < nb) ? (i <= r ? A[static_cast<int64_t>(k0 + r) * n + k0 + i] : 0.0) : (r == i ? 1.0 : 0.0);
#pragma unroll
    for (int r = 0; r < CH_NB; ++r) L[r][i] = in[r];
  }
  __syncthreads();
  double row[CH_NB];
#pragma unroll
  for (int c = 0; c < CH_NB; ++c) row[c] = L[i][c];
  int bad = 0;
  double rp_own = 1.0;  // lane j: 1 / pivot j
#pragma unroll
  for (int j = 0; j < CH_NB; ++j) {
    col[i] = row[j];
    KVX_COMPILER_FENCE();
    double cj[CH_NB];  // column j as published (entries j..63 read)
#pragma unroll
    for (int c = j & ~1; c < CH_NB; c += 2) {
      const double2 v = *reinterpret_cast<const double2*>(&col[c]);
      cj[c] = v.x;
      cj[c + 1] = v.y;
    }
    KVX_COMPILER_FENCE();
    const double d = cj[j];
    const bool ok = d > 0.0;
    if (j < nb && !ok) bad = 1;
    const double piv = sqrt(ok ? d : 1.0);
    const double rp = 1.0 / piv;
    rp_own = i == j ? rp : rp_own;
    row[j] = i == j ? piv : (i > j ? row[j] * rp : row[j]);
    // L[c][j] = cj[c] * rp: the reciprocal joins this lane's multiplier
    const double t = row[j] * rp;
#pragma unroll
    for (int c = j + 1; c < CH_NB; ++c) row[c] = fma(-t, cj[c], row[c]);
  }
  if (bad && i == 0) *flag = 1;
  __syncthreads();  // every lane has read its row of the input
#pragma unroll
  for (int c = 0; c < CH_NB; ++c) L[i][c] = (c <= i) ? row[c] : 0.0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < CH_NB; ++r)
    if (i < nb && r < nb && r >= i) A[static_cast<int64_t>(k0 + r) * n + k0 + i] = L[r][i];
  // inverse: lane c forms column c (entries above the diagonal come out 0)
  double x[CH_NB];
#pragma unroll
  for (int r = 0; r < CH_NB; ++r) {
    // the sum taken positive and subtracted once (written as repeated
    // fma(-l, x, v), this loop takes the compiler minutes)
    double a = 0.0;
#pragma unroll
    for (int q = 0; q < r; ++q) a = fma(L[r][q], x[q], a);
    x[r] = (((r == i) ? 1.0 : 0.0) - a) * readlane_f64(rp_own, r);
  }
#pragma unroll
  for (int r = 0; r < CH_NB; ++r) linv[r * CH_NB + i] = (r < nb && i < nb) ? x[r] : 0.0;
}

// C[M x N] -= A * B (overwrite = 0) or C = A * B (overwrite = 1) in fp64 on
// matrix cores, for a batch of problems (blockIdx.z; the operands of problem
// z start bsa, bsb, bsc elements after those of problem z-1), with
// A(m,k) = A[m*sam + k*sak] and B(k,n) = B[k*sbk + n*sbn].  Block tiles of
// BT x BT; 2 x NWN waves, each from MFMA 16x16x4 fp64 blocks; K in
// chunks of 16 through LDS (global elements are read along the operand's
// unit-stride index and kept in that order: [k][m] / [k][n], or [m][k] /
// [n][k] for an operand read along k; rows padded against bank conflicts of
// the stores and of the fragment reads); the next chunk is read
// into registers while the current one is multiplied.  A workgroup reads all
// of its A rows and B columns before it writes its tile, so C may alias A when
// N <= BT or B when M <= BT.  lower_only forms only the tiles on and
// below the diagonal (the grid holds just those).
struct DgArgs {
  int32_t M, N, K;
  const double* A;
  int64_t sam, sak, bsa;
  const double* B;
  int64_t sbk, sbn, bsb;
  double* C;
  int64_t ldc, bsc;
  int32_t lower_only, overwrite;
};
constexpr int DG_BK = 16;

// BT = 64: 64 x 64 block tiles (small products), the updated C tile read
// before the K loop; BT = 128: 128 x 128 block tiles (large products, long
// K).  2 x NWN waves, each a (BT / 2) x (BT / NWN) wave tile.
// AK / BK: A / B read along k (unit stride in k), else along m / n.
template <int BT, int NWN>
constexpr int dg_min_waves() {
  return BT == 64 ? 3 : (NWN == 4 ? 4 : 2);
}
template <int BT, int NWN, bool AK, bool BK>
__global__ __attribute__((amdgpu_flat_work_group_size(128 * NWN, 128 * NWN),
                          amdgpu_waves_per_eu(dg_min_waves<BT, NWN>(), 8))) void
dgemm_kernel(const DgArgs g) {
  constexpr int NT = 128 * NWN;        // threads
  constexpr int LD = BT + 16;          // [k][m] rows (doubles): 16-lane row pieces in distinct banks
  // an operand read along k is kept [m][k] with an odd row stride: a thread's
  // store is then contiguous with its neighbours' and the 16 rows of a
  // fragment read start in distinct bank pairs (kept [k][m], its transposing
  // stores put 8 lanes on one bank pair)
  constexpr int LDK = DG_BK + 1;
  constexpr int NQ = BT * DG_BK / NT;  // elements of A (and of B) per thread and chunk
  constexpr int WTM = BT / 2, WTN = BT / NWN;
  constexpr int NFM = WTM / 16, NFN = WTN / 16;  // MFMA blocks per wave along m and n
  constexpr bool PRE_C = BT == 64;
  int32_t bm = blockIdx.y, bn = blockIdx.x;
  if (g.lower_only) {
    // blockIdx.x enumerates only the tiles on and below the diagonal, row by
    // row (row bm holds min(bm + 1, column tiles) of them), so consecutive
    // workgroups, which go to different XCDs, share the work evenly
    const int32_t nbn = (g.N + BT - 1) / BT;
    int32_t t = blockIdx.x;
    bm = 0;
    for (;;) {
      const int32_t w = bm + 1 < nbn ? bm + 1 : nbn;
      if (t < w) break;
      t -= w;
      ++bm;
    }
    bn = t;
  }
  __shared__ double As[AK ? BT : DG_BK][AK ? LDK : LD];
  __shared__ double Bs[BK ? BT : DG_BK][BK ? LDK : LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int32_t m0 = bm * BT, n0 = bn * BT;
  const double* A = g.A + blockIdx.z * g.bsa;
  const double* B = g.B + blockIdx.z * g.bsb;
  double* C = g.C + blockIdx.z * g.bsc;
  constexpr bool a_k = AK, b_k = BK;
  // this thread's elements of a chunk: fixed row / column, k offset 0..15,
  // as byte offsets from the chunk's first k (one 32-bit register each, the
  // chunk's base a uniform pointer); every operand of one problem holds at
  // most KVX_MAX_FIT_FEATURES^2 = 2^28 elements, so they fit
  uint32_t oa[NQ], ob[NQ];
  uint32_t va = 0, vb = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = tid + NT * q;
    const int ma = a_k ? (e >> 4) : (e % BT), ka = a_k ? (e & 15) : (e / BT);
    if (m0 + ma < g.M) va |= 1u << q;
    oa[q] = static_cast<uint32_t>(((m0 + ma) * g.sam + ka * g.sak) * 8);
    const int nb_ = b_k ? (e >> 4) : (e % BT), kb = b_k ? (e & 15) : (e / BT);
    if (n0 + nb_ < g.N) vb |= 1u << q;
    ob[q] = static_cast<uint32_t>(((n0 + nb_) * g.sbn + kb * g.sbk) * 8);
  }
  double av[NQ], bv[NQ];
  // buffer loads: the per-lane offset above plus the chunk's uniform offset;
  // an element outside the operand takes an offset past the resource's end,
  // which reads zero without a memory access
  constexpr uint32_t OOB = 0x7ffffff8u;
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(A, OOB), rb = buf_rsrc(B, OOB);
  auto load = [&](int32_t k0) {
    const uint32_t sa = static_cast<uint32_t>(static_cast<int64_t>(k0) * g.sak * 8);
    const uint32_t sb = static_cast<uint32_t>(static_cast<int64_t>(k0) * g.sbk * 8);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = tid + NT * q;
      const int ka = a_k ? (e & 15) : (e / BT), kb = b_k ? (e & 15) : (e / BT);
      const uint32_t pa = ((va >> q) & 1u) && k0 + ka < g.K ? oa[q] : OOB;
      const uint32_t pb = ((vb >> q) & 1u) && k0 + kb < g.K ? ob[q] : OOB;
      av[q] = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(ra, pa, sa, 0));
      bv[q] = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(rb, pb, sb, 0));
    }
  };
  // element r of lane l: row l/16 + 4r, column l%16 of its 16 x 16 block
  auto row_of = [&](int i, int r) { return m0 + wm * WTM + i * 16 + (lane >> 4) + 4 * r; };
  auto col_of = [&](int j) { return n0 + wn * WTN + j * 16 + (lane & 15); };

  f64x4 acc[NFM][NFN], cv[PRE_C ? NFM : 1][PRE_C ? NFN : 1];
#pragma unroll
  for (int i = 0; i < NFM; ++i)
#pragma unroll
    for (int j = 0; j < NFN; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  load(0);
  if constexpr (PRE_C) {
#pragma unroll
    for (int i = 0; i < NFM; ++i)
#pragma unroll
      for (int j = 0; j < NFN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t m = row_of(i, r), n = col_of(j);
          cv[i][j][r] = (!g.overwrite && m < g.M && n < g.N) ? C[m * g.ldc + n] : 0.0;
        }
  }
  for (int32_t k0 = 0; k0 < g.K; k0 += DG_BK) {
    __syncthreads();  // the previous chunk's fragment reads are done
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = tid + NT * q;
      if constexpr (AK)
        As[e >> 4][e & 15] = av[q];
      else
        As[e / BT][e % BT] = av[q];
      if constexpr (BK)
        Bs[e >> 4][e & 15] = bv[q];
      else
        Bs[e / BT][e % BT] = bv[q];
    }
    __syncthreads();
    if (k0 + DG_BK < g.K) load(k0 + DG_BK);
#pragma unroll
    for (int k4 = 0; k4 < DG_BK; k4 += 4) {
      // operands of MFMA 16x16x4: lane l holds A[l%16][l/16] and B[l/16][l%16]
      const int kr = k4 + (lane >> 4);
      double a[NFM], b[NFN];
#pragma unroll
      for (int i = 0; i < NFM; ++i) {
        const int m = wm * WTM + i * 16 + (lane & 15);
        if constexpr (AK)
          a[i] = As[m][kr];
        else
          a[i] = As[kr][m];
      }
#pragma unroll
      for (int j = 0; j < NFN; ++j) {
        const int nn = wn * WTN + j * 16 + (lane & 15);
        if constexpr (BK)
          b[j] = Bs[nn][kr];
        else
          b[j] = Bs[kr][nn];
      }
#pragma unroll
      for (int i = 0; i < NFM; ++i)
#pragma unroll
        for (int j = 0; j < NFN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < NFM; ++i)
#pragma unroll
    for (int j = 0; j < NFN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int32_t m = row_of(i, r), n = col_of(j);
        if (m < g.M && n < g.N) {
          double c_old;
          if constexpr (PRE_C)
            c_old = cv[i][j][r];
          else
            c_old = g.overwrite ? 0.0 : C[m * g.ldc + n];
          C[m * g.ldc + n] = g.overwrite ? acc[i][j][r] : c_old - acc[i][j][r];
        }
      }
}

// w_out[f][o] = W[f][o] rounded to fp32 (both row-major [f_in][f_out]).
__global__ __launch_bounds__(256) void fit_store_kernel(const double* __restrict__ W, int64_t n,
                                                        float* __restrict__ w_out) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    w_out[i] = static_cast<float>(W[i]);
}

// The bias b[o] = mean_y[o] - sum_f mean_x[f] W[f][o] in two passes with a
// fixed order: workgroup (g, q) adds rows q*rows_per .. of its 256 columns
// into partial[q][o]; then the BI_CHUNKS partials are added in chunk order.
constexpr int BI_CHUNKS = 64;
__global__ __launch_bounds__(256) void fit_bias_part_kernel(const double* __restrict__ W, int32_t f_in, int32_t f_out,
                                                            const double* __restrict__ sx, double inv_n,
                                                            int32_t rows_per, double* __restrict__ partial) {
  const int32_t o = blockIdx.x * 256 + threadIdx.x;
  if (o >= f_out) return;
  const int32_t f1 = min(f_in, static_cast<int32_t>((blockIdx.y + 1) * rows_per));
  double a = 0.0;
  for (int32_t f = blockIdx.y * rows_per; f < f1; ++f) a += sx[f] * inv_n * W[static_cast<int64_t>(f) * f_out + o];
  partial[static_cast<int64_t>(blockIdx.y) * f_out + o] = a;
}

__global__ __launch_bounds__(256) void fit_bias_final_kernel(const double* __restrict__ partial, int32_t f_out,
                                                             const double* __restrict__ sy, double inv_n,
                                                             float* __restrict__ b_out) {
  const int32_t o = blockIdx.x * 256 + threadIdx.x;
  if (o >= f_out) return;
  double a = 0.0;
  for (int q = 0; q < BI_CHUNKS; ++q) a += partial[static_cast<int64_t>(q) * f_out + o];
  b_out[o] = static_cast<float>(sy[o] * inv_n - a);
}

// Outputs of one fitted problem: w_out (row-major fp32 [f_in][f_out]) and,
// when b_out is not null, the bias.  partial: BI_CHUNKS * f_out doubles of
// scratch.
static int fit_output(hipStream_t s, const double* W, int32_t f_in, int32_t f_out, float* w_out, float* b_out,
                      const double* sx, const double* sy, double inv_n, double* partial) {
  const int64_t n = static_cast<int64_t>(f_in) * f_out;
  fit_store_kernel<<<static_cast<unsigned>(ceil_div(n, 256) < 8192 ? ceil_div(n, 256) : 8192), 256, 0, s>>>(W, n, w_out);
  KVX_LAUNCH_CHECK();
  if (b_out) {
    const int32_t rows_per = static_cast<int32_t>(ceil_div(f_in, BI_CHUNKS));
    fit_bias_part_kernel<<<dim3(static_cast<unsigned>(ceil_div(f_out, 256)), BI_CHUNKS), 256, 0, s>>>(
        W, f_in, f_out, sx, inv_n, rows_per, partial);
    fit_bias_final_kernel<<<static_cast<unsigned>(ceil_div(f_out, 256)), 256, 0, s>>>(partial, f_out, sy, inv_n, b_out);
    KVX_LAUNCH_CHECK();
  }
  return KVX_OK;
}

// Inverse of each 256-wide diagonal block of the factor (for the block
// triangular solves), assembled per problem (blockIdx.y) from the 64-wide
// inverse factors: first the diagonal 64 x 64 pieces are placed.
constexpr int SV_NB = 256;  // block of the triangular solves
__global__ __launch_bounds__(256) void place_linv_kernel(const double* __restrict__ linv, double* __restrict__ xinv,
                                                         int64_t bs) {
  const int32_t kb = blockIdx.x;
  const double* src = linv + blockIdx.y * bs + static_cast<int64_t>(kb) * CH_NB * CH_NB;
  double* dst = xinv + blockIdx.y * bs + static_cast<int64_t>(kb / 4) * SV_NB * SV_NB +
                static_cast<int64_t>(kb % 4) * CH_NB * (SV_NB + 1);
  for (int e = threadIdx.x; e < CH_NB * CH_NB; e += 256) dst[(e / CH_NB) * SV_NB + e % CH_NB] = src[e];
}

__global__ __launch_bounds__(256) void fill_f64_kernel(double* __restrict__ p, int64_t n, int64_t bs, double v) {
  double* q = p + blockIdx.y * bs;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n; e += static_cast<int64_t>(gridDim.x) * 256)
    q[e] = v;
}

__global__ __launch_bounds__(256) void copy_f64_kernel(const double* __restrict__ src, double* __restrict__ dst,
                                                       int64_t n, int64_t bs) {
  const double* a = src + blockIdx.y * bs;
  double* b = dst + blockIdx.y * bs;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n; e += static_cast<int64_t>(gridDim.x) * 256)
    b[e] = a[e];
}

// ---------------------------------------------------------------- host side

// Workspace: the Gram partials (shared by the problems, which are
// accumulated one after the other), then per problem G, C, column sums,
// lambda and the inverse diagonal factors, then one flag per problem.
struct FitWs {
  float* part;
  double* csp;  // column-sum partials [CS_CHUNKS][max(f_in, f_out)]
  double *G, *C, *sx, *sy, *lam, *linv, *xinv, *zbuf;
  int64_t bs;  // doubles between the per-problem areas
  int64_t oG, oC, oSx, oSy, oLam, oLinv, oXinv, oZbuf;
  int32_t* flags;
  size_t bytes;
};

// with_part = false: no Gram split partials (the Gram from runs writes G and
// C directly).
static FitWs fit_layout(int32_t count, int32_t f_in, int32_t f_out, void* base, bool with_part = true) {
  FitWs w{};
  Carve c(base);
  w.part = with_part ? c.take<float>(static_cast<size_t>(GR_MAX_SPLIT) * f_in * (static_cast<size_t>(f_in) + f_out))
                     : nullptr;
  w.csp = c.take<double>(static_cast<size_t>(CS_CHUNKS) * (f_in > f_out ? f_in : f_out));
  const int64_t nb_total = ceil_div(f_in, CH_NB);
  auto up = [](int64_t v) { return (v + 31) / 32 * 32; };  // 256-byte sub-areas
  w.oG = 0;
  w.oC = w.oG + up(static_cast<int64_t>(f_in) * f_in);
  w.oSx = w.oC + up(static_cast<int64_t>(f_in) * f_out);
  w.oSy = w.oSx + up(f_in);
  w.oLam = w.oSy + up(f_out);
  w.oLinv = w.oLam + up(4);
  w.oXinv = w.oLinv + up(nb_total * CH_NB * CH_NB);
  const int64_t n_outer = ceil_div(f_in, SV_NB);
  w.oZbuf = w.oXinv + up(n_outer * SV_NB * SV_NB);
  const int64_t zb = static_cast<int64_t>(SV_NB) * f_out;
  w.bs = w.oZbuf + up(zb > CH_NB * 3 * CH_NB ? zb : CH_NB * 3 * CH_NB);
  double* area = c.take<double>(static_cast<size_t>(count) * w.bs);
  if (area) {
    w.G = area + w.oG;
    w.C = area + w.oC;
    w.sx = area + w.oSx;
    w.sy = area + w.oSy;
    w.lam = area + w.oLam;
    w.linv = area + w.oLinv;
    w.xinv = area + w.oXinv;
    w.zbuf = area + w.oZbuf;
  }
  w.flags = c.take<int32_t>(static_cast<size_t>(count) + 64);
  w.bytes = c.used + 256;
  return w;
}

size_t fit_ws_bytes(int32_t count, int32_t f_in, int32_t f_out) { return fit_layout(count, f_in, f_out, nullptr).bytes; }

static unsigned grid_for(int64_t n) {
  int64_t b = ceil_div(n, 256);
  if (b > 16384) b = 16384;
  return static_cast<unsigned>(b < 1 ? 1 : b);
}

static int dgemm(hipStream_t s, int32_t count, int32_t M, int32_t N, int32_t K, const double* A, int64_t sam,
                 int64_t sak, const double* B, int64_t sbk, int64_t sbn, double* C, int64_t ldc, int64_t bs,
                 int32_t lower_only, int32_t overwrite, int64_t bsb = -1) {
  DgArgs g{M, N, K, A, sam, sak, bs, B, sbk, sbn, bsb < 0 ? bs : bsb, C, ldc, bs, lower_only, overwrite};
  // 128-wide tiles for large in-place-free products with a long K (aliasing
  // of C with A or B is only used with one 64-wide tile along that side)
  const bool ak = sak == 1 && sam != 1, bk = sbk == 1 && sbn != 1;
  const bool big = M >= 128 && N >= 128 && K >= 128;
  const int bt = big ? 128 : 64;
  const int64_t nbm = ceil_div(M, bt), nbn = ceil_div(N, bt);
  int64_t n_lower = 0;  // tiles on and below the diagonal
  for (int64_t bm = 0; bm < nbm; ++bm) n_lower += bm + 1 < nbn ? bm + 1 : nbn;
  const dim3 grid = lower_only ? dim3(static_cast<unsigned>(n_lower), 1, static_cast<unsigned>(count))
                               : dim3(static_cast<unsigned>(nbn), static_cast<unsigned>(nbm),
                                      static_cast<unsigned>(count));
#define KVX_DG(BT_, NWN_, A_, B_) dgemm_kernel<BT_, NWN_, A_, B_><<<grid, 128 * NWN_, 0, s>>>(g)
  if (big) {
    constexpr int W = 4;  // 8 waves of 64 x 32 (4 waves of 64 x 64 ran 3-4% slower)
    if (ak) { if (bk) KVX_DG(128, W, true, true); else KVX_DG(128, W, true, false); }
    else { if (bk) KVX_DG(128, W, false, true); else KVX_DG(128, W, false, false); }
  } else {
    if (ak) { if (bk) KVX_DG(64, 2, true, true); else KVX_DG(64, 2, true, false); }
    else { if (bk) KVX_DG(64, 2, false, true); else KVX_DG(64, 2, false, false); }
  }
#undef KVX_DG
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// Blocked Cholesky A = L L^T (lower, in place) of `count` problems of order
// n; problem z's A, linv, xinv and zbuf sit z * bs doubles after problem 0's.
// The diagonal kernel leaves the inverse of each 64-wide factor in linv, so
// each panel solve is an in-place product with it.  Right-looking by
// 256-column panels: inside a panel, each 64-wide block is factored, its
// panel solved and only the panel's remaining columns updated; the trailing
// matrix right of the panel is updated once per panel with K = 256, so it is
// read and written n/256 rather than n/64 times.  Afterwards xinv holds the
// inverses of the 256-wide diagonal blocks for the triangular solves:
// X_bb = L_bb^-1 (placed), then for each lower block row b,
// X[b, 0:b] = -L_bb^-1 (L[b, 0:b] X[0:b, 0:b]).  Entries strictly above the
// diagonal of A are left with partial updates (only the lower triangle is
// the factor).  A non-positive pivot sets flags[z].
// When the call's problems fill the chip with the products (see
// factor_left), the factorisation runs left-looking instead: each panel is
// first reduced by all columns left of it in one product (K = p0), and
// nothing right of the panel is touched, so each column block is read and
// written once by those products rather than once per panel to its left.
static bool factor_left(int32_t count, int32_t n) {
  return static_cast<int64_t>(count) * ceil_div(n, 128) * (SV_NB / 128) >= 384;
}

static int chol_factor(hipStream_t s, int32_t count, double* A, int32_t n, int64_t bs, double* linv, double* xinv,
                       double* zbuf, int32_t* flags) {
  const int32_t nb_total = static_cast<int32_t>(ceil_div(n, CH_NB));
  const int32_t n_outer = static_cast<int32_t>(ceil_div(n, SV_NB));
  const bool left = factor_left(count, n);
  for (int32_t I = 0; I < n_outer; ++I) {
    const int32_t p0 = I * SV_NB;
    const int32_t pn = min(SV_NB, n - p0);
    if (left && p0 > 0) {
      // A[p0:n][p0:p0+pn] -= A[p0:n][0:p0] A[p0:p0+pn][0:p0]^T (lower part)
      const double* Lr = A + static_cast<int64_t>(p0) * n;
      double* Ct = A + static_cast<int64_t>(p0) * n + p0;
      if (int st = dgemm(s, count, n - p0, pn, p0, Lr, n, 1, Lr, 1, n, Ct, n, bs, 1, 0)) return st;
    }
    for (int32_t k0 = p0; k0 < p0 + pn; k0 += CH_NB) {
      const int32_t nb = min(CH_NB, n - k0);
      double* li = linv + static_cast<int64_t>(k0 / CH_NB) * CH_NB * CH_NB;
      potrf_diag_kernel<<<static_cast<unsigned>(count), 64, 0, s>>>(A, bs, n, k0, nb, flags, li, bs);
      KVX_LAUNCH_CHECK();
      const int32_t rest = n - k0 - nb;
      if (rest <= 0) continue;
      // panel: P = P L_kk^-T (in place, one 64-column tile)
      double* P = A + static_cast<int64_t>(k0 + nb) * n + k0;
      if (int st = dgemm(s, count, rest, nb, nb, P, n, 1, li, 1, CH_NB, P, n, bs, 0, 1)) return st;
      // the panel's remaining columns: A[r][c] -= P[r] . P[c], c < p0 + pn
      const int32_t pw = p0 + pn - (k0 + nb);
      if (pw > 0) {
        double* Ct = A + static_cast<int64_t>(k0 + nb) * n + k0 + nb;
        if (int st = dgemm(s, count, rest, pw, nb, P, n, 1, P, 1, n, Ct, n, bs, 1, 0)) return st;
      }
    }
    // trailing lower update right of the panel, K = the panel's width
    const int32_t rest = n - p0 - pn;
    if (!left && rest > 0) {
      const double* PI = A + static_cast<int64_t>(p0 + pn) * n + p0;
      double* Ct = A + static_cast<int64_t>(p0 + pn) * n + p0 + pn;
      if (int st = dgemm(s, count, rest, rest, pn, PI, n, 1, PI, 1, n, Ct, n, bs, 1, 0)) return st;
    }
  }
  const dim3 fill_grid(static_cast<unsigned>(ceil_div(static_cast<int64_t>(n_outer) * SV_NB * SV_NB, 256 * 8)),
                       static_cast<unsigned>(count));
  fill_f64_kernel<<<fill_grid, 256, 0, s>>>(xinv, static_cast<int64_t>(n_outer) * SV_NB * SV_NB, bs, 0.0);
  KVX_LAUNCH_CHECK();
  place_linv_kernel<<<dim3(static_cast<unsigned>(nb_total), static_cast<unsigned>(count)), 256, 0, s>>>(linv, xinv,
                                                                                                      bs);
  KVX_LAUNCH_CHECK();
  for (int32_t I = 0; I < n_outer; ++I) {
    const int32_t k0 = I * SV_NB;
    const int32_t nb = min(SV_NB, n - k0);
    double* X = xinv + static_cast<int64_t>(I) * SV_NB * SV_NB;
    for (int32_t b = 1; b * CH_NB < nb; ++b) {
      const int32_t sb = min(CH_NB, nb - b * CH_NB);
      const int32_t wb = b * CH_NB;
      // T = L[b, 0:b] X[0:b, 0:b] (in zbuf, row stride 3 * 64)
      if (int st = dgemm(s, count, sb, wb, wb, A + static_cast<int64_t>(k0 + wb) * n + k0, n, 1, X, SV_NB, 1, zbuf,
                         3 * CH_NB, bs, 0, 1))
        return st;
      // X[b, 0:b] = 0 - L_bb^-1 T
      const double* li = linv + static_cast<int64_t>(I * 4 + b) * CH_NB * CH_NB;
      if (int st = dgemm(s, count, sb, wb, sb, li, CH_NB, 1, zbuf, 3 * CH_NB, 1, X + static_cast<int64_t>(wb) * SV_NB,
                         SV_NB, bs, 0, 0))
        return st;
    }
  }
  return KVX_OK;
}

static int copy_back(hipStream_t s, int32_t count, const double* src, double* dst, int64_t n, int64_t bs) {
  copy_f64_kernel<<<dim3(static_cast<unsigned>(ceil_div(n, 256 * 8)), static_cast<unsigned>(count)), 256, 0, s>>>(
      src, dst, n, bs);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// Right-looking L Z = C (C [n][nrhs], row stride nrhs) by 256-row blocks:
// Z_I = X_II C_I, then the rows below are updated,
// so the right-hand sides are read and written n/256 times.  zbuf holds
// 256 x nrhs doubles.
static int chol_forward_right(hipStream_t s, int32_t count, const double* A, int32_t n, int64_t bs, const double* xinv,
                        double* zbuf, double* C, int32_t nrhs) {
  const int32_t n_outer = static_cast<int32_t>(ceil_div(n, SV_NB));
  for (int32_t I = 0; I < n_outer; ++I) {
    const int32_t k0 = I * SV_NB;
    const int32_t nb = min(SV_NB, n - k0);
    const double* X = xinv + static_cast<int64_t>(I) * SV_NB * SV_NB;
    double* CI = C + static_cast<int64_t>(k0) * nrhs;
    if (int st = dgemm(s, count, nb, nrhs, nb, X, SV_NB, 1, CI, nrhs, 1, zbuf, nrhs, bs, 0, 1)) return st;
    if (int st = copy_back(s, count, zbuf, CI, static_cast<int64_t>(nb) * nrhs, bs)) return st;
    const int32_t rest = n - k0 - nb;
    if (rest > 0) {
      const double* Lb = A + static_cast<int64_t>(k0 + nb) * n + k0;
      if (int st = dgemm(s, count, rest, nrhs, nb, Lb, n, 1, zbuf, nrhs, 1, CI + static_cast<int64_t>(nb) * nrhs, nrhs,
                         bs, 0, 0))
        return st;
    }
  }
  return KVX_OK;
}

// Right-looking L^T W = Z (W_I = X_II^T Z_I, then the rows above are updated).
static int chol_backward_right(hipStream_t s, int32_t count, const double* A, int32_t n, int64_t bs, const double* xinv,
                         double* zbuf, double* C, int32_t nrhs) {
  const int32_t n_outer = static_cast<int32_t>(ceil_div(n, SV_NB));
  for (int32_t I = n_outer - 1; I >= 0; --I) {
    const int32_t k0 = I * SV_NB;
    const int32_t nb = min(SV_NB, n - k0);
    const double* X = xinv + static_cast<int64_t>(I) * SV_NB * SV_NB;
    double* CI = C + static_cast<int64_t>(k0) * nrhs;
    if (int st = dgemm(s, count, nb, nrhs, nb, X, 1, SV_NB, CI, nrhs, 1, zbuf, nrhs, bs, 0, 1)) return st;
    if (int st = copy_back(s, count, zbuf, CI, static_cast<int64_t>(nb) * nrhs, bs)) return st;
    if (k0 > 0) {
      // Z[0..k0) -= L[k0..k0+nb)[0..k0)^T W_I
      const double* Lr = A + static_cast<int64_t>(k0) * n;
      if (int st = dgemm(s, count, k0, nrhs, nb, Lr, 1, n, zbuf, nrhs, 1, C, nrhs, bs, 0, 0)) return st;
    }
  }
  return KVX_OK;
}

// Gram and cross products of one problem into its G and C.
// Left-looking L Z = C (C [n][nrhs], row stride nrhs) by 256-row blocks: block I is first reduced by every
// solved block above it in one product (C_I -= L[I, 0:I] Z[0:I], K = the
// rows solved so far), then Z_I = X_II C_I.  Each block of right-hand sides
// is read and written twice, and the long-K product keeps the fp64 matrix
// cores fed.  zbuf holds 256 x nrhs doubles.
static int chol_forward_left(hipStream_t s, int32_t count, const double* A, int32_t n, int64_t bs, const double* xinv,
                        double* zbuf, double* C, int32_t nrhs) {
  const int32_t n_outer = static_cast<int32_t>(ceil_div(n, SV_NB));
  for (int32_t I = 0; I < n_outer; ++I) {
    const int32_t k0 = I * SV_NB;
    const int32_t nb = min(SV_NB, n - k0);
    const double* X = xinv + static_cast<int64_t>(I) * SV_NB * SV_NB;
    double* CI = C + static_cast<int64_t>(k0) * nrhs;
    if (k0 > 0) {
      const double* Lb = A + static_cast<int64_t>(k0) * n;  // L[k0 .. k0+nb)[0 .. k0)
      if (int st = dgemm(s, count, nb, nrhs, k0, Lb, n, 1, C, nrhs, 1, CI, nrhs, bs, 0, 0)) return st;
    }
    if (int st = dgemm(s, count, nb, nrhs, nb, X, SV_NB, 1, CI, nrhs, 1, zbuf, nrhs, bs, 0, 1)) return st;
    if (int st = copy_back(s, count, zbuf, CI, static_cast<int64_t>(nb) * nrhs, bs)) return st;
  }
  return KVX_OK;
}

// Left-looking L^T W = Z from the last block: Z_I -= L[below, I]^T
// W[below] in one product, then W_I = X_II^T Z_I.
static int chol_backward_left(hipStream_t s, int32_t count, const double* A, int32_t n, int64_t bs, const double* xinv,
                         double* zbuf, double* C, int32_t nrhs) {
  const int32_t n_outer = static_cast<int32_t>(ceil_div(n, SV_NB));
  for (int32_t I = n_outer - 1; I >= 0; --I) {
    const int32_t k0 = I * SV_NB;
    const int32_t nb = min(SV_NB, n - k0);
    const double* X = xinv + static_cast<int64_t>(I) * SV_NB * SV_NB;
    double* CI = C + static_cast<int64_t>(k0) * nrhs;
    const int32_t rest = n - k0 - nb;
    if (rest > 0) {
      // A[m][k] = L[k0 + nb + k][k0 + m]; B = the solved rows below
      const double* Lc = A + static_cast<int64_t>(k0 + nb) * n + k0;
      if (int st = dgemm(s, count, nb, nrhs, rest, Lc, 1, n, C + static_cast<int64_t>(k0 + nb) * nrhs, nrhs, 1, CI,
                         nrhs, bs, 0, 0))
        return st;
    }
    if (int st = dgemm(s, count, nb, nrhs, nb, X, 1, SV_NB, CI, nrhs, 1, zbuf, nrhs, bs, 0, 1)) return st;
    if (int st = copy_back(s, count, zbuf, CI, static_cast<int64_t>(nb) * nrhs, bs)) return st;
  }
  return KVX_OK;
}

// The triangular solves for the factor of chol_factor, in place.  The
// left-looking order reads and writes each block of right-hand sides twice
// but runs one product of 256 x nrhs per problem and block; it is used when
// the problems of the call give those products enough tiles to fill the
// chip, else the right-looking order, whose updates span every row below.
static bool solve_left(int32_t count, int32_t nrhs) {
  return static_cast<int64_t>(count) * (SV_NB / 128) * ceil_div(nrhs, 128) >= 512;
}

static int chol_forward(hipStream_t s, int32_t count, const double* A, int32_t n, int64_t bs, const double* xinv,
                        double* zbuf, double* C, int32_t nrhs) {
  return solve_left(count, nrhs) ? chol_forward_left(s, count, A, n, bs, xinv, zbuf, C, nrhs)
                                 : chol_forward_right(s, count, A, n, bs, xinv, zbuf, C, nrhs);
}

static int chol_backward(hipStream_t s, int32_t count, const double* A, int32_t n, int64_t bs, const double* xinv,
                         double* zbuf, double* C, int32_t nrhs) {
  return solve_left(count, nrhs) ? chol_backward_left(s, count, A, n, bs, xinv, zbuf, C, nrhs)
                                 : chol_backward_right(s, count, A, n, bs, xinv, zbuf, C, nrhs);
}

// The Grams of `batch` problems of one shape from bf16 rows, in as few
// launches as the partials' room allows: problem b reads x + b x_batch and
// y + b y_batch (f_out = 0: X^T X only) and writes its G and C b bs doubles
// after problem 0's; `part` has room for part_cap floats of split partials.
static int gram_batch(const uint16_t* x, int64_t ldx, int64_t x_batch, const uint16_t* y, int64_t ldy,
                      int64_t y_batch, int64_t n_rows, int32_t f_in, int32_t f_out, int32_t batch, float* part,
                      int64_t part_cap, double* G, double* C, int64_t bs, hipStream_t s) {
  const int64_t per_split = static_cast<int64_t>(f_in) * (static_cast<int64_t>(f_in) + f_out);
  const int64_t fit = part_cap / per_split;  // problems whose single-split partials fit at once
  if (fit < 1) return KVX_ERR_WORKSPACE;
  if (batch > fit) {
    for (int32_t b0 = 0; b0 < batch; b0 += static_cast<int32_t>(fit)) {
      const int32_t nb = static_cast<int32_t>(std::min<int64_t>(fit, batch - b0));
      if (int st = gram_batch(x + b0 * x_batch, ldx, x_batch, y ? y + b0 * y_batch : nullptr, ldy, y_batch, n_rows,
                              f_in, f_out, nb, part, part_cap, G + b0 * bs, C ? C + b0 * bs : nullptr, bs, s))
        return st;
    }
    return KVX_OK;
  }
  GramArgs g{};
  g.x = x;
  g.y = y;
  g.ldx = ldx;
  g.ldy = ldy;
  g.n_rows = n_rows;
  g.f_in = f_in;
  g.f_out = f_out;
  g.nbi = static_cast<int32_t>(ceil_div(f_in, GR_T));
  g.nbc = static_cast<int32_t>(ceil_div(f_out, GR_T));
  g.n_g = g.nbi * (g.nbi + 1) / 2;
  g.n_c = g.nbi * g.nbc;
  g.batch = batch;
  g.x_batch = x_batch;
  g.y_batch = y_batch;
  // row splits: the fewest that fill the persistent grid best (fewer
  // partials to add up, longer K loops), each at least one step long, as
  // many as the partials' room holds
  const int cus = device_cu_count();
  const int64_t tiles = static_cast<int64_t>(batch) * (g.n_g + g.n_c);
  const int64_t cap_split = std::min<int64_t>(GR_MAX_SPLIT, part_cap / (per_split * batch));
  int64_t split = 1;
  double best = 0.0;
  for (int64_t sp = 1; sp <= cap_split; ++sp) {
    const int64_t items = sp * tiles;
    const double eff = static_cast<double>(items) / static_cast<double>(ceil_div(items, cus) * cus);
    if (eff > best + 1e-9) {
      best = eff;
      split = sp;
    }
  }
  const int64_t max_split = ceil_div(n_rows, GR_BK);
  if (split > max_split) split = max_split > 0 ? max_split : 1;
  g.rows_per_split = ceil_div(ceil_div(n_rows, split), GR_BK) * GR_BK;
  if (g.rows_per_split > 0) split = ceil_div(n_rows, g.rows_per_split);
  g.split = static_cast<int32_t>(split);
  // a split's rows are addressed with 32-bit byte offsets
  if (g.rows_per_split * 2 * (ldx > ldy ? ldx : ldy) >= (1LL << 31)) return KVX_ERR_UNSUPPORTED;
  g.part = part;
  const int64_t items = split * tiles;
  const unsigned grid = static_cast<unsigned>(items < cus ? items : cus);
  gram_kernel<<<grid, GR_THREADS, 0, s>>>(g);
  KVX_LAUNCH_CHECK();
  const int64_t nbi = ceil_div(f_in, RD_T), nbc = ceil_div(f_out, RD_T);
  gram_reduce_kernel<<<dim3(static_cast<unsigned>(nbi * (nbi + 1) / 2 + nbi * nbc), static_cast<unsigned>(batch)),
                       256, 0, s>>>(part, g.split, f_in, f_out, G, C, bs);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

static int gram_one(const void* x, int64_t ldx, const void* y, int64_t ldy, int32_t in_f32, int64_t n_rows,
                    int32_t f_in, int32_t f_out, float* part, double* G, double* C, hipStream_t s) {
  if (in_f32) {
    gram_f32_kernel<<<grid_for(static_cast<int64_t>(f_in) * (f_in + f_out)), 256, 0, s>>>(
        static_cast<const float*>(x), ldx, static_cast<const float*>(y), ldy, n_rows, f_in, f_out, G, C);
    KVX_LAUNCH_CHECK();
    return KVX_OK;
  }
  return gram_batch(static_cast<const uint16_t*>(x), ldx, 0, static_cast<const uint16_t*>(y), ldy, 0, n_rows, f_in,
                    f_out, 1, part, static_cast<int64_t>(GR_MAX_SPLIT) * f_in * (static_cast<int64_t>(f_in) + f_out),
                    G, C, 0, s);
}

int launch_fit(int32_t count, const void* const* x, int64_t ldx, const void* const* y, int64_t ldy, int32_t in_f32,
               int64_t n_rows, int32_t f_in, int32_t f_out, double lam_abs, double lam_rel, int32_t fit_intercept,
               float* const* w_out, float* const* b_out, int32_t* status, void* ws, hipStream_t s) {
  const FitWs w = fit_layout(count, f_in, f_out, ws);
  const int64_t bs = w.bs;
  if (int st = launch_fill_i32(w.flags, count, 0, s)) return st;
  const double inv_n = n_rows > 0 ? 1.0 / static_cast<double>(n_rows) : 0.0;

  // 1. Gram and cross products, centring and lambda, problem by problem
  for (int32_t z = 0; z < count; ++z) {
    double* G = w.G + z * bs;
    double* C = w.C + z * bs;
    double* sx = w.sx + z * bs;
    double* sy = w.sy + z * bs;
    if (int st = gram_one(x[z], ldx, y[z], ldy, in_f32, n_rows, f_in, f_out, w.part, G, C, s)) return st;
    if (fit_intercept) {
      if (int st = colsum(x[z], ldx, n_rows, f_in, in_f32, w.csp, sx, s)) return st;
      if (int st = colsum(y[z], ldy, n_rows, f_out, in_f32, w.csp, sy, s)) return st;
      center_kernel<<<grid_for(static_cast<int64_t>(f_in) * (f_in + f_out)), 256, 0, s>>>(G, C, sx, sy, f_in, f_out,
                                                                                          inv_n, 0);
      KVX_LAUNCH_CHECK();
    }
    lambda_kernel<<<1, 256, 0, s>>>(G, f_in, lam_abs, lam_rel, w.lam + z * bs);
    KVX_LAUNCH_CHECK();
  }

  // 2. Cholesky and the two block triangular solves of all problems at once
  if (int st = chol_factor(s, count, w.G, f_in, bs, w.linv, w.xinv, w.zbuf, w.flags)) return st;
  if (int st = chol_forward(s, count, w.G, f_in, bs, w.xinv, w.zbuf, w.C, f_out)) return st;
  if (int st = chol_backward(s, count, w.G, f_in, bs, w.xinv, w.zbuf, w.C, f_out)) return st;

  // 3. outputs
  for (int32_t z = 0; z < count; ++z) {
    if (int st = fit_output(s, w.C + z * bs, f_in, f_out, w_out[z], fit_intercept ? b_out[z] : nullptr,
                            w.sx + z * bs, w.sy + z * bs, inv_n, w.csp))
      return st;
  }

  std::vector<int32_t> host_flags(static_cast<size_t>(count), 0);
  KVX_HIP_TRY(hipMemcpyAsync(host_flags.data(), w.flags, sizeof(int32_t) * count, hipMemcpyDeviceToHost, s));
  KVX_HIP_TRY(hipStreamSynchronize(s));
  int result = KVX_OK;
  for (int32_t z = 0; z < count; ++z) {
    if (status) status[z] = host_flags[z] ? KVX_ERR_NOT_SPD : KVX_OK;
    if (host_flags[z]) result = KVX_ERR_NOT_SPD;
  }
  return result;
}

// ---------------------------------------------------------------- fit from the caches
//
// Every receiver layer and role of a model pair from the calibration caches
// (see gram_runs_kernel for the Gram from the alignment's runs).  Problems are
// ordered role by role (K, then V), receiver layer within; the fp64 solve is
// the one of launch_fit, all problems at once.

__global__ __launch_bounds__(256) void lambda_batched_kernel(double* __restrict__ G, int64_t bs, int32_t f_in,
                                                             double lam_abs, double lam_rel,
                                                             double* __restrict__ lam_out) {
  // problem blockIdx.x: the same fixed summation order as lambda_kernel
  G += blockIdx.x * bs;
  __shared__ double red[256];
  double sum = 0.0;
  for (int32_t i = threadIdx.x; i < f_in; i += 256) sum += G[static_cast<int64_t>(i) * f_in + i];
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double lam = lam_abs + lam_rel * red[0] / static_cast<double>(f_in);
  for (int32_t i = threadIdx.x; i < f_in; i += 256) G[static_cast<int64_t>(i) * f_in + i] += lam;
  if (threadIdx.x == 0) lam_out[blockIdx.x * bs] = lam;
}

// The Gram-from-runs part of a workspace (both fits from the caches).
constexpr int SG_CHUNKS = 64;  // run chunks of the weighted feature sums
struct RunsWs {
  Runs runs;
  void* runs_scratch;
  int32_t* glist;
  int32_t* taps;
  GrrKey* keys;        // distinct lower G tiles (at most one per problem and tile)
  GrrDest* dests;      // their consumers (one per problem and tile)
  uint16_t* xu;
  uint16_t* xg;
  uint16_t* qp;
  double* sigma;       // [L_S][row]: sum_u c_u x_u of every sender layer (one role)
  double* sigma_part;  // [L_S][SG_CHUNKS][row]: its per-chunk partials
  float2* tab_send;    // (cos, sin) per sender position and pair, when the sender keys are rotated
  float2* tab_recv;    // the same for the receiver's (target) keys
  int64_t u_cap, g_cap;  // row capacities of xu (and half of qp) and xg
};

// Sized for the worst case of n_recv runs of one token: U <= n_recv, and the
// bit-group rows sum_u popcount(c_u) <= sum_u c_u = n_recv, plus padding.
static RunsWs runs_layout(const FitcShape& sh, Carve& c) {
  RunsWs w{};
  const int32_t n = sh.n_recv;
  w.runs.uniq = c.take<int32_t>(n);
  w.runs.run_begin = c.take<int32_t>(static_cast<size_t>(n) + 1);
  w.runs.recv_to_uniq = c.take<int32_t>(n);
  w.runs.n_uniq = c.take<int32_t>(64);
  w.runs_scratch = c.take<char>(runs_ws_bytes(n));
  w.u_cap = ceil_div(n, GR_BK) * GR_BK;
  w.g_cap = ceil_div(static_cast<int64_t>(n) + static_cast<int64_t>(GRR_MAX_GROUPS) * GRR_PAD, GRR_PAD) * GRR_PAD;
  w.glist = c.take<int32_t>(static_cast<size_t>(w.g_cap));
  w.taps = c.take<int32_t>(static_cast<size_t>(sh.recv_layers) * sh.n_taps);
  const int64_t nb = ceil_div(sh.f_in, GR_T);
  w.keys = c.take<GrrKey>(static_cast<size_t>(sh.recv_layers) * (nb * (nb + 1) / 2));
  w.dests = c.take<GrrDest>(static_cast<size_t>(sh.recv_layers) * (nb * (nb + 1) / 2));
  w.xu = c.take<uint16_t>(static_cast<size_t>(sh.send_layers) * w.u_cap * sh.row);
  w.xg = c.take<uint16_t>(static_cast<size_t>(sh.send_layers) * w.g_cap * sh.row);
  w.qp = c.take<uint16_t>(static_cast<size_t>(sh.recv_layers) * 2 * w.u_cap * sh.f_out);
  w.sigma = c.take<double>(static_cast<size_t>(sh.send_layers) * sh.row);
  w.sigma_part = c.take<double>(static_cast<size_t>(sh.send_layers) * SG_CHUNKS * sh.row);
  if (sh.send_rope > 0.0) w.tab_send = c.take<float2>(static_cast<size_t>(sh.n_send) * (sh.send_hd / 2));
  if (sh.recv_rope > 0.0) w.tab_recv = c.take<float2>(static_cast<size_t>(sh.n_recv) * (sh.recv_hd / 2));
  return w;
}

struct FitcWs {
  FitWs fit;
  RunsWs r;
  size_t bytes;
};

static FitcWs fitc_layout(const FitcShape& sh, void* base) {
  FitcWs w{};
  w.fit = fit_layout(sh.count, sh.f_in, sh.f_out, base, false);
  Carve c(base);
  c.used = w.fit.bytes;
  w.r = runs_layout(sh, c);
  w.bytes = c.used + 256;
  return w;
}

size_t fitc_ws_bytes(const FitcShape& sh) { return fitc_layout(sh, nullptr).bytes; }

int64_t fitc_max_rows(const FitcShape& sh) {
  const FitcWs w = fitc_layout(sh, nullptr);
  return w.r.g_cap > 2 * w.r.u_cap ? w.r.g_cap : 2 * w.r.u_cap;
}

// The bit groups of the run lengths c_u (from run_begin, host), largest bit
// first: group j holds the runs with bit j of c_u set (j < 15), group 15 the
// runs with c_u >= 2^15, each c_u >> 15 times; each group padded with -1 to
// whole GRR_PAD rows.
static void fitc_groups(const std::vector<int32_t>& rb, int32_t n_runs, std::vector<int32_t>& list,
                        GramRunsArgs& g) {
  list.clear();
  g.n_groups = 0;
  for (int j = GRR_MAX_GROUPS - 1; j >= 0; --j) {
    const size_t start = list.size();
    for (int32_t u = 0; u < n_runs; ++u) {
      const int32_t cu = rb[static_cast<size_t>(u) + 1] - rb[static_cast<size_t>(u)];
      const int32_t reps = j == GRR_MAX_GROUPS - 1 ? (cu >> (GRR_MAX_GROUPS - 1)) : ((cu >> j) & 1);
      for (int32_t q = 0; q < reps; ++q) list.push_back(u);
    }
    if (list.size() == start) continue;
    while (list.size() % GRR_PAD) list.push_back(-1);
    g.grp_exp[g.n_groups] = j;
    g.grp_end[g.n_groups] = static_cast<int32_t>(list.size() / GRR_PAD);
    ++g.n_groups;
  }
}

// The distinct lower tiles of G over all problems of a role: tile (bi, bj),
// bi >= bj, of receiver layer l pairs sender layer taps[l][bi 256 / row] at
// row offset bi 256 mod row with the same for bj; keys ordered by (layers,
// offsets) with the larger (layer, offset) on the row side, so consecutive
// items share their row panel.
static void fitc_keys(const FitcShape& sh, const int32_t* taps, std::vector<GrrKey>& keys,
                      std::vector<GrrDest>& dests) {
  const int32_t nb = static_cast<int32_t>(ceil_div(sh.f_in, GR_T));
  std::map<std::array<int32_t, 4>, std::vector<GrrDest>> m;
  for (int32_t l = 0; l < sh.recv_layers; ++l)
    for (int32_t bi = 0; bi < nb; ++bi)
      for (int32_t bj = 0; bj <= bi; ++bj) {
        const std::array<int32_t, 2> a{taps[l * sh.n_taps + bi * GR_T / sh.row], bi * GR_T % sh.row};
        const std::array<int32_t, 2> b{taps[l * sh.n_taps + bj * GR_T / sh.row], bj * GR_T % sh.row};
        if (a >= b)
          m[{a[0], a[1], b[0], b[1]}].push_back(GrrDest{l, bi, bj, 0});
        else
          m[{b[0], b[1], a[0], a[1]}].push_back(GrrDest{l, bi, bj, 1});
      }
  keys.clear();
  dests.clear();
  for (const auto& kv : m) {
    keys.push_back(GrrKey{kv.first[0], kv.first[1], kv.first[2], kv.first[3], static_cast<int32_t>(dests.size()),
                          static_cast<int32_t>(kv.second.size()), 0, 0});
    dests.insert(dests.end(), kv.second.begin(), kv.second.end());
  }
}

// Run-length-weighted column sums of the distinct rows of every sender layer
// (sum_u c_u x_u, n times the feature means of that layer's taps), in two
// passes: each one-wave workgroup sums SG_CHUNKS-th of the runs for 512
// columns (8 per lane, 16-byte loads), fp64 partials written per chunk; then
// the chunks are added in order.
__global__ __launch_bounds__(64) void fitc_sigma_part_kernel(const uint16_t* __restrict__ xu, int64_t xu_layer,
                                                             int32_t row, const int32_t* __restrict__ run_begin,
                                                             int32_t n_runs, double* __restrict__ part) {
  const int32_t c0 = (blockIdx.x * 64 + threadIdx.x) * 8;
  const int64_t sl = blockIdx.z;
  const int32_t per = (n_runs + SG_CHUNKS - 1) / SG_CHUNKS;
  const int32_t u0 = blockIdx.y * per;
  const int32_t u1 = min(n_runs, u0 + per);
  if (c0 >= row) return;
  const uint16_t* col = xu + sl * xu_layer + c0;
  double acc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = 0.0;
  for (int32_t u = u0; u < u1; ++u) {
    const double c = static_cast<double>(run_begin[u + 1] - run_begin[u]);
    const u32x4 q = *reinterpret_cast<const u32x4*>(col + static_cast<int64_t>(u) * row);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += c * static_cast<double>(bf16lo(q[e]));
      acc[2 * e + 1] += c * static_cast<double>(bf16hi(q[e]));
    }
  }
  double* out = part + (sl * SG_CHUNKS + blockIdx.y) * row + c0;
#pragma unroll
  for (int v = 0; v < 8; ++v) out[v] = acc[v];
}

__global__ __launch_bounds__(256) void fitc_sigma_final_kernel(const double* __restrict__ part, int32_t row,
                                                               double* __restrict__ sigma) {
  const int64_t sl = blockIdx.y;
  const int32_t f = blockIdx.x * 256 + threadIdx.x;
  if (f >= row) return;
  double a = 0.0;
  for (int q = 0; q < SG_CHUNKS; ++q) a += part[(sl * SG_CHUNKS + q) * row + f];
  sigma[sl * row + f] = a;
}

// sx of problem z (receiver layer z - z0): tap t's row of sigma.
__global__ __launch_bounds__(256) void fitc_sx_kernel(const double* __restrict__ sigma, int32_t row,
                                                      const int32_t* __restrict__ taps, int32_t n_taps,
                                                      double* __restrict__ sx, int64_t bs) {
  const int32_t l = blockIdx.y;
  const int32_t f = blockIdx.x * 256 + threadIdx.x;
  if (f >= n_taps * row) return;
  sx[l * bs + f] = sigma[static_cast<int64_t>(taps[l * n_taps + f / row]) * row + f % row];
}

// The moments from the runs for every role (problems role by role, receiver
// layer within; problem z's G and C at z * bs): the runs, their bit groups and
// the shared tiles once, then per role the distinct and bit-group rows of
// every sender layer, the run sums of the targets and one Gram launch.  With
// sx non-null also each problem's feature column sums (n times the means).
static int gram_from_runs(const FitcShape& sh, const RunsWs& w, const void* const* send_role,
                          const void* const* recv_role, const int32_t* map, const int32_t* taps_host, double* G,
                          double* C, double* sx, int64_t bs, hipStream_t s) {
  // 1. runs of the alignment; their lengths on the host for the bit groups
  if (int st = launch_runs(map, sh.n_recv, sh.n_send, w.runs, w.runs_scratch, s)) return st;
  int32_t n_runs = 0;
  KVX_HIP_TRY(hipMemcpyAsync(&n_runs, w.runs.n_uniq, sizeof(int32_t), hipMemcpyDeviceToHost, s));
  KVX_HIP_TRY(hipStreamSynchronize(s));
  if (n_runs < 1 || n_runs > sh.n_recv) return KVX_ERR_HIP;
  std::vector<int32_t> rb(static_cast<size_t>(n_runs) + 1);
  KVX_HIP_TRY(hipMemcpyAsync(rb.data(), w.runs.run_begin, sizeof(int32_t) * rb.size(), hipMemcpyDeviceToHost, s));
  KVX_HIP_TRY(hipStreamSynchronize(s));
  GramRunsArgs g{};
  std::vector<int32_t> list;
  fitc_groups(rb, n_runs, list, g);
  if (static_cast<int64_t>(list.size()) > w.g_cap) return KVX_ERR_HIP;
  const int32_t u_pad = static_cast<int32_t>(ceil_div(n_runs, GR_BK) * GR_BK);
  KVX_HIP_TRY(hipMemcpyAsync(w.glist, list.data(), sizeof(int32_t) * list.size(), hipMemcpyHostToDevice, s));

  g.row = sh.row;
  g.xg_rows = static_cast<int32_t>(list.size());
  g.u_pad = u_pad;
  g.xg_layer = static_cast<int64_t>(g.xg_rows) * sh.row;
  g.xu_layer = static_cast<int64_t>(u_pad) * sh.row;
  g.qp_layer = 2LL * u_pad * sh.f_out;
  g.xg = w.xg;
  g.xu = w.xu;
  g.qp = w.qp;
  g.taps = w.taps;
  g.n_taps = sh.n_taps;
  g.n_problems = sh.recv_layers;
  g.f_in = sh.f_in;
  g.f_out = sh.f_out;
  g.nbi = static_cast<int32_t>(ceil_div(sh.f_in, GR_T));
  g.nbc = static_cast<int32_t>(ceil_div(sh.f_out, GR_T));
  g.n_g = g.nbi * (g.nbi + 1) / 2;
  g.n_c = g.nbi * g.nbc;
  g.bs = bs;
  KVX_HIP_TRY(hipMemcpyAsync(w.taps, taps_host, sizeof(int32_t) * sh.recv_layers * sh.n_taps, hipMemcpyHostToDevice,
                             s));
  std::vector<GrrKey> keys;
  std::vector<GrrDest> dests;
  fitc_keys(sh, taps_host, keys, dests);
  KVX_HIP_TRY(hipMemcpyAsync(w.keys, keys.data(), sizeof(GrrKey) * keys.size(), hipMemcpyHostToDevice, s));
  KVX_HIP_TRY(hipMemcpyAsync(w.dests, dests.data(), sizeof(GrrDest) * dests.size(), hipMemcpyHostToDevice, s));
  g.keys = w.keys;
  g.dests = w.dests;
  g.n_keys = static_cast<int32_t>(keys.size());
  if (sh.key_role >= 0 && sh.send_rope > 0.0)
    if (int st = launch_rope_table(w.tab_send, sh.n_send, sh.send_hd, sh.send_rope, s)) return st;
  if (sh.key_role >= 0 && sh.recv_rope > 0.0)
    if (int st = launch_rope_table(w.tab_recv, sh.n_recv, sh.recv_hd, sh.recv_rope, s)) return st;

  // 2. per role: the distinct rows and the bit-group rows of every sender
  // layer, the run sums of the targets, then the Gram of all its problems
  // (keys stored rotated are turned back on the way: the sender's at the
  // sender position, the targets at the receiver position)
  const int cus = device_cu_count();
  for (int32_t r = 0; r < sh.n_roles; ++r) {
    const uint16_t* xs = static_cast<const uint16_t*>(send_role[r]);
    const uint16_t* ys = static_cast<const uint16_t*>(recv_role[r]);
    const bool rot_x = r == sh.key_role && sh.send_rope > 0.0;
    const bool rot_y = r == sh.key_role && sh.recv_rope > 0.0;
    const int64_t send_layer = static_cast<int64_t>(sh.n_send) * sh.row;
    const unsigned gx_u = static_cast<unsigned>(std::min<int64_t>(ceil_div(g.xu_layer / 8, 256), 4096));
    const unsigned gx_g = static_cast<unsigned>(std::min<int64_t>(ceil_div(g.xg_layer / 8, 256), 4096));
    const dim3 grid_u(gx_u, static_cast<unsigned>(sh.send_layers)), grid_g(gx_g, static_cast<unsigned>(sh.send_layers));
    if (rot_x) {
      fitc_gather_kernel<true><<<grid_u, 256, 0, s>>>(xs, send_layer, sh.row, w.runs.uniq, nullptr, n_runs, u_pad,
                                                      w.xu, g.xu_layer, w.tab_send, sh.send_hd);
      fitc_gather_kernel<true><<<grid_g, 256, 0, s>>>(xs, send_layer, sh.row, w.runs.uniq, w.glist, 0, g.xg_rows,
                                                      w.xg, g.xg_layer, w.tab_send, sh.send_hd);
    } else {
      fitc_gather_kernel<false><<<grid_u, 256, 0, s>>>(xs, send_layer, sh.row, w.runs.uniq, nullptr, n_runs, u_pad,
                                                       w.xu, g.xu_layer, nullptr, 0);
      fitc_gather_kernel<false><<<grid_g, 256, 0, s>>>(xs, send_layer, sh.row, w.runs.uniq, w.glist, 0, g.xg_rows,
                                                       w.xg, g.xg_layer, nullptr, 0);
    }
    KVX_LAUNCH_CHECK();
    const dim3 grid_q(
        static_cast<unsigned>(std::min<int64_t>(ceil_div(static_cast<int64_t>(u_pad) * sh.f_out / 8, 256), 4096)),
        static_cast<unsigned>(sh.recv_layers));
    const int64_t y_layer = static_cast<int64_t>(sh.n_recv) * sh.f_out;
    if (rot_y)
      fitc_target_sums_kernel<true><<<grid_q, 256, 0, s>>>(ys, y_layer, sh.f_out, w.runs.run_begin, n_runs, u_pad,
                                                           w.qp, g.qp_layer, w.tab_recv, sh.recv_hd);
    else
      fitc_target_sums_kernel<false><<<grid_q, 256, 0, s>>>(ys, y_layer, sh.f_out, w.runs.run_begin, n_runs, u_pad,
                                                            w.qp, g.qp_layer, nullptr, 0);
    KVX_LAUNCH_CHECK();
    GramRunsArgs gr = g;
    const int64_t z0 = static_cast<int64_t>(r) * sh.recv_layers;
    gr.G = G + z0 * bs;
    gr.C = C + z0 * bs;
    const int64_t items = g.n_keys + static_cast<int64_t>(sh.recv_layers) * g.n_c;
    gram_runs_kernel<<<static_cast<unsigned>(items < cus ? items : cus), GR_THREADS, 0, s>>>(gr);
    KVX_LAUNCH_CHECK();
    if (sx) {
      // rows are whole 16-byte pieces: row is a multiple of 256
      fitc_sigma_part_kernel<<<dim3(static_cast<unsigned>(ceil_div(sh.row, 512)), SG_CHUNKS,
                                    static_cast<unsigned>(sh.send_layers)),
                               64, 0, s>>>(w.xu, g.xu_layer, sh.row, w.runs.run_begin, n_runs, w.sigma_part);
      fitc_sigma_final_kernel<<<dim3(static_cast<unsigned>(ceil_div(sh.row, 256)),
                                     static_cast<unsigned>(sh.send_layers)),
                                256, 0, s>>>(w.sigma_part, sh.row, w.sigma);
      KVX_LAUNCH_CHECK();
      fitc_sx_kernel<<<dim3(static_cast<unsigned>(ceil_div(sh.f_in, 256)), static_cast<unsigned>(sh.recv_layers)),
                       256, 0, s>>>(w.sigma, sh.row, w.taps, sh.n_taps, sx + z0 * bs, bs);
      KVX_LAUNCH_CHECK();
    }
  }
  return KVX_OK;
}

int launch_fit_caches(const FitcShape& sh, const void* const* send_role, const void* const* recv_role,
                      const int32_t* map, const int32_t* taps_host, double lam_abs, double lam_rel,
                      float* const* w_role, int32_t* status, void* ws, hipStream_t s) {
  const FitcWs w = fitc_layout(sh, ws);
  const int64_t bs = w.fit.bs;
  if (int st = launch_fill_i32(w.fit.flags, sh.count, 0, s)) return st;
  if (int st = gram_from_runs(sh, w.r, send_role, recv_role, map, taps_host, w.fit.G, w.fit.C, nullptr, bs, s))
    return st;
  lambda_batched_kernel<<<static_cast<unsigned>(sh.count), 256, 0, s>>>(w.fit.G, bs, sh.f_in, lam_abs, lam_rel,
                                                                        w.fit.lam);
  KVX_LAUNCH_CHECK();

  // 3. Cholesky and the two block triangular solves of all problems at once
  if (int st = chol_factor(s, sh.count, w.fit.G, sh.f_in, bs, w.fit.linv, w.fit.xinv, w.fit.zbuf, w.fit.flags))
    return st;
  if (int st = chol_forward(s, sh.count, w.fit.G, sh.f_in, bs, w.fit.xinv, w.fit.zbuf, w.fit.C, sh.f_out)) return st;
  if (int st = chol_backward(s, sh.count, w.fit.G, sh.f_in, bs, w.fit.xinv, w.fit.zbuf, w.fit.C, sh.f_out)) return st;

  // 4. outputs [f_in][f_out] per problem
  const int64_t nw = static_cast<int64_t>(sh.f_in) * sh.f_out;
  for (int32_t z = 0; z < sh.count; ++z) {
    float* out = w_role[z / sh.recv_layers] + static_cast<int64_t>(z % sh.recv_layers) * nw;
    fit_store_kernel<<<grid_for(nw), 256, 0, s>>>(w.fit.C + z * bs, nw, out);
    KVX_LAUNCH_CHECK();
  }

  std::vector<int32_t> host_flags(static_cast<size_t>(sh.count), 0);
  KVX_HIP_TRY(hipMemcpyAsync(host_flags.data(), w.fit.flags, sizeof(int32_t) * sh.count, hipMemcpyDeviceToHost, s));
  KVX_HIP_TRY(hipStreamSynchronize(s));
  int result = KVX_OK;
  for (int32_t z = 0; z < sh.count; ++z) {
    if (status) status[z] = host_flags[z] ? KVX_ERR_NOT_SPD : KVX_OK;
    if (host_flags[z]) result = KVX_ERR_NOT_SPD;
  }
  return result;
}

// ---------------------------------------------------------------- Recolor
//
// "Prefill-Free Cross-Family KV Cache Transfer ..." (Key Contributions 2,
// Methodology 3): the moment-matched map whitens both feature spaces, aligns
// the whitened spaces by an orthogonal Procrustes solution and restores the
// receiver's covariance and mean:
//   W = A_x Q A_y^-1,  b = mean_y - mean_x W,  A^T S A = I,
//   Q = polar factor of the whitened cross-covariance A_x^T S_xy A_y.
// W does not depend on which whitening A is used (A R for an orthogonal R
// gives the same W), so the Cholesky factors S_xx = L_x L_x^T and
// S_yy = L_y L_y^T serve: A_x = L_x^-T, A_y^-1 = L_y^T, and
//   M = L_x^-1 S_xy L_y^-T,  Q = M (M^T M)^-1/2,  W = L_x^-T Q L_y^T.
// Moments are kept as n times the covariances (the factor cancels in W and
// in the relative regulariser rho * trace / F added to each diagonal).  The
// inverse square root of S = M^T M comes from the coupled Newton-Schulz
// iteration Y <- Y T, Z <- T Z of third order, T = (15 I - 10 P + 3 P^2) / 8
// with P = Z Y (x^-1/2 to second order about 1; the second-order step
// T = (3 I - P) / 2 took about 1.4 times as many steps for one more product
// fewer), started at Y = S / c, Z = I with c = min(1.1 lam, ||S||_F), lam a
// power-iteration estimate of the largest eigenvalue (the scalar step
// x <- x p(x)^2 converges to 1 for x in (0, 2.3), and each step multiplies a
// small eigenvalue of S / c by (15/8)^2): Z -> (S / c)^-1/2.  All products
// are fp64 on matrix cores, every problem of the call at once; the host
// reads ||T - I||_F per problem after each step.  T - I = -(P - I)/2 to first
// order and the step takes an error e of P to about e^3, so once
// ||T - I||_F <= RC_TOL (spectral error of P at most about 2e-4) the step
// being applied brings P to within about 1e-11 of I, far below the fp32
// rounding of the maps, and the iteration ends with it, with no further step
// to confirm it.

constexpr int NS_BLOCKS = 64;        // workgroups per problem of the middle step
constexpr int RC_MAX_ITERS = 100;
constexpr int RC_POWER = 12;         // power steps for the largest eigenvalue of M^T M
constexpr double RC_TOL = 1e-4;      // ||T - I||_F after which this step's update is the last
// below this, a step that gains < 4x is the rounding floor (a step from
// ||T - I||_F <= 1e-3 that still converges gains far more)
constexpr double RC_FLOOR = 1e-3;
// ||(S / c)^-1/2||_F above this: M is numerically rank-deficient (fewer
// distinct calibration rows than outputs, or outputs unrelated to the
// features in some direction), so the polar factor is not determined
constexpr double RC_ZMAX = 1e6;

__global__ __launch_bounds__(256) void identity_kernel(double* __restrict__ p, int32_t n, int64_t bs) {
  double* q = p + blockIdx.y * bs;
  const int64_t total = static_cast<int64_t>(n) * n;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256)
    q[e] = (e / n == e % n) ? 1.0 : 0.0;
}

// Entries strictly above the diagonal set to zero (the factor is the lower
// triangle).
__global__ __launch_bounds__(256) void zero_upper_kernel(double* __restrict__ p, int32_t n, int64_t bs) {
  double* q = p + blockIdx.y * bs;
  const int64_t total = static_cast<int64_t>(n) * n;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256)
    if (e % n > e / n) q[e] = 0.0;
}

// ||S||_F of each problem in a fixed summation order: NS_BLOCKS workgroups
// per problem sum the squares of interleaved elements, then the partials are
// added in block order.
__global__ __launch_bounds__(256) void frob_part_kernel(const double* __restrict__ S, int32_t n, int64_t bs,
                                                        double* __restrict__ part) {
  const double* q = S + blockIdx.y * bs;
  __shared__ double red[256];
  const int64_t total = static_cast<int64_t>(n) * n;
  double a = 0.0;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total; e += NS_BLOCKS * 256)
    a += q[e] * q[e];
  red[threadIdx.x] = a;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.y * NS_BLOCKS + blockIdx.x] = red[0];
}

__global__ __launch_bounds__(64) void frob_final_kernel(const double* __restrict__ part, int64_t bs,
                                                        double* __restrict__ out) {
  if (threadIdx.x != 0) return;
  double a = 0.0;
  for (int b = 0; b < NS_BLOCKS; ++b) a += part[blockIdx.x * NS_BLOCKS + b];
  out[blockIdx.x * bs] = sqrt(a);
}

// out[z * bs] = ||S_z||_F; part holds count * NS_BLOCKS doubles
static int frob(hipStream_t s, int32_t count, const double* S, int32_t n, int64_t bs, double* part, double* out) {
  frob_part_kernel<<<dim3(NS_BLOCKS, static_cast<unsigned>(count)), 256, 0, s>>>(S, n, bs, part);
  frob_final_kernel<<<static_cast<unsigned>(count), 64, 0, s>>>(part, bs, out);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// Symmetric from its lower triangle: every entry above the diagonal of each
// problem's n x n matrix is set to its mirror below.  One workgroup per 64 x
// 64 block on or above the diagonal reads the mirror block row by row into
// LDS and writes the block row by row (a diagonal block only above its
// diagonal); the blocks it reads are never written.
__global__ __launch_bounds__(256) void sym_from_lower_kernel(double* __restrict__ P, int32_t n, int64_t bs) {
  __shared__ double tile[RD_T][RD_T + 1];
  double* q = P + blockIdx.y * bs;
  const int32_t nb = (n + RD_T - 1) / RD_T;
  int32_t t = blockIdx.x, bi = 0, rowlen = nb;
  while (t >= rowlen) {
    t -= rowlen;
    ++bi;
    --rowlen;
  }
  const int32_t bj = bi + t;  // target block (bi, bj), bi <= bj; source (bj, bi)
  for (int e = threadIdx.x; e < RD_T * RD_T; e += 256) {
    const int r = e / RD_T, c = e % RD_T;
    const int32_t m = bj * RD_T + r, k = bi * RD_T + c;
    tile[r][c] = (m < n && k < n) ? q[static_cast<int64_t>(m) * n + k] : 0.0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < RD_T * RD_T; e += 256) {
    const int r = e / RD_T, c = e % RD_T;
    const int32_t i = bi * RD_T + r, j = bj * RD_T + c;
    if (i < n && j < n && j > i) q[static_cast<int64_t>(i) * n + j] = tile[c][r];
  }
}

static int sym_from_lower(hipStream_t s, int32_t count, double* P, int32_t n, int64_t bs) {
  const int32_t nb = static_cast<int32_t>(ceil_div(n, RD_T));
  sym_from_lower_kernel<<<dim3(static_cast<unsigned>(nb * (nb + 1) / 2), static_cast<unsigned>(count)), 256, 0, s>>>(
      P, n, bs);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// p *= c^power with c = scal of the problem.
__global__ __launch_bounds__(256) void scale_kernel(double* __restrict__ p, int64_t n, int64_t bs,
                                                    const double* __restrict__ scal, double power) {
  double* q = p + blockIdx.y * bs;
  const double f = pow(scal[blockIdx.y * bs], power);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n; e += static_cast<int64_t>(gridDim.x) * 256)
    q[e] *= f;
}

// Start vector of the power iteration (deterministic, no special direction):
// v_i = 0.5 + frac(0.6180339887 (i + 1)).
__global__ __launch_bounds__(256) void power_start_kernel(double* __restrict__ v, int32_t n, int64_t bs) {
  double* q = v + blockIdx.x * bs;
  for (int32_t i = threadIdx.x; i < n; i += 256) {
    const double t = 0.6180339887498949 * static_cast<double>(i + 1);
    q[i] = 0.5 + (t - floor(t));
  }
}

// One workgroup per problem: lam = ||y|| (fixed summation order), v = y / lam.
__global__ __launch_bounds__(256) void power_norm_kernel(const double* __restrict__ y, double* __restrict__ v,
                                                         int32_t n, int64_t bs, double* __restrict__ lam) {
  y += blockIdx.x * bs;
  v += blockIdx.x * bs;
  __shared__ double red[256];
  double a = 0.0;
  for (int32_t i = threadIdx.x; i < n; i += 256) a += y[i] * y[i];
  red[threadIdx.x] = a;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double nrm = sqrt(red[0]);
  const double inv = nrm > 0.0 ? 1.0 / nrm : 0.0;
  for (int32_t i = threadIdx.x; i < n; i += 256) v[i] = y[i] * inv;
  if (threadIdx.x == 0) lam[blockIdx.x * bs] = nrm;
}

// Scale of the polar iteration: c = min(1.1 lam, ||S||_F) with lam the power
// iteration's estimate of the largest eigenvalue (never above it for a unit
// vector, close to it after the steps run); ||S||_F bounds it from above.
__global__ void polar_scale_kernel(double* __restrict__ scal, int64_t bs) {
  double* q = scal + blockIdx.x * bs;
  const double c = 1.1 * q[2];
  if (threadIdx.x == 0) q[0] = (c > 0.0 && c < q[0]) ? c : q[0];
}

// Middle of a third-order Newton-Schulz step: from P = Z Y and Q = P^2,
// T = (15 I - 10 P + 3 Q) / 8 in place of P (x^-1/2 to second order about
// x = 1, at x = P); each workgroup writes the sum of (T - I)^2 over its share
// (NaN propagates) to dev[problem][workgroup].
__global__ __launch_bounds__(256) void ns_mid_kernel(double* __restrict__ P, const double* __restrict__ Q,
                                                      int32_t n, int64_t bs, double* __restrict__ dev) {
  double* p = P + blockIdx.y * bs;
  const double* q = Q + blockIdx.y * bs;
  __shared__ double red[256];
  const int64_t total = static_cast<int64_t>(n) * n;
  double m = 0.0;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total; e += NS_BLOCKS * 256) {
    const double id = (e / n == e % n) ? 1.0 : 0.0;
    const double t = (15.0 * id - 10.0 * p[e] + 3.0 * q[e]) * 0.125;
    p[e] = t;
    m += (t - id) * (t - id);
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) dev[blockIdx.y * NS_BLOCKS + blockIdx.x] = red[0];
}

struct RcWs {
  float* part;
  double* csp;
  double *G, *C, *sx, *sy, *lam, *linvx, *xinvx, *zbuf, *Gy, *linvy, *xinvy, *E, *M, *ns[4], *scal;
  int64_t bs;
  double* dev;
  int32_t* flags;
  size_t bytes;
};

static RcWs recolor_layout(int32_t count, int32_t f_in, int32_t f_out, void* base) {
  RcWs w{};
  Carve c(base);
  w.part = c.take<float>(static_cast<size_t>(GR_MAX_SPLIT) * f_in * (static_cast<size_t>(f_in) + f_out));
  w.csp = c.take<double>(static_cast<size_t>(CS_CHUNKS) * (f_in > f_out ? f_in : f_out));
  int64_t o = 0;
  auto take = [&](int64_t n) {
    const int64_t at = o;
    o += (n + 31) / 32 * 32;  // 256-byte sub-areas
    return at;
  };
  const int64_t fi = f_in, fo = f_out;
  const int64_t zb = static_cast<int64_t>(SV_NB) * fo;
  const int64_t oG = take(fi * fi), oC = take(fi * fo), oSx = take(fi), oSy = take(fo), oLam = take(4);
  const int64_t oLx = take(ceil_div(fi, CH_NB) * CH_NB * CH_NB), oXx = take(ceil_div(fi, SV_NB) * SV_NB * SV_NB);
  const int64_t oZ = take(zb > CH_NB * 3 * CH_NB ? zb : CH_NB * 3 * CH_NB);
  const int64_t oGy = take(fo * fo), oLy = take(ceil_div(fo, CH_NB) * CH_NB * CH_NB);
  const int64_t oXy = take(ceil_div(fo, SV_NB) * SV_NB * SV_NB), oE = take(fo * fo), oM = take(fi * fo);
  int64_t oN[4];
  for (int i = 0; i < 4; ++i) oN[i] = take(fo * fo);
  const int64_t oS = take(4);
  w.bs = o;
  double* area = c.take<double>(static_cast<size_t>(count) * w.bs);
  if (area) {
    w.G = area + oG;
    w.C = area + oC;
    w.sx = area + oSx;
    w.sy = area + oSy;
    w.lam = area + oLam;
    w.linvx = area + oLx;
    w.xinvx = area + oXx;
    w.zbuf = area + oZ;
    w.Gy = area + oGy;
    w.linvy = area + oLy;
    w.xinvy = area + oXy;
    w.E = area + oE;
    w.M = area + oM;
    for (int i = 0; i < 4; ++i) w.ns[i] = area + oN[i];
    w.scal = area + oS;
  }
  w.dev = c.take<double>(static_cast<size_t>(count) * NS_BLOCKS);
  w.flags = c.take<int32_t>(static_cast<size_t>(count) + 64);
  w.bytes = c.used + 256;
  return w;
}

size_t recolor_ws_bytes(int32_t count, int32_t f_in, int32_t f_out) {
  return recolor_layout(count, f_in, f_out, nullptr).bytes;
}

static int recolor_solve(RcWs& w, int32_t count, int32_t f_in, int32_t f_out, double inv_n, float* const* w_out,
                         float* const* b_out, int32_t* status, int32_t* iters, hipStream_t s);

int launch_recolor(int32_t count, const void* const* x, int64_t ldx, const void* const* y, int64_t ldy,
                   int32_t in_f32, int64_t n_rows, int32_t f_in, int32_t f_out, double rho_x, double rho_y,
                   float* const* w_out, float* const* b_out, int32_t* status, int32_t* iters, void* ws,
                   hipStream_t s) {
  RcWs w = recolor_layout(count, f_in, f_out, ws);
  const int64_t bs = w.bs;
  if (int st = launch_fill_i32(w.flags, count, 0, s)) return st;
  const double inv_n = n_rows > 0 ? 1.0 / static_cast<double>(n_rows) : 0.0;
  const int64_t fo2 = static_cast<int64_t>(f_out) * f_out;
  const dim3 grid_o2(grid_for(fo2 / 8 + 1), static_cast<unsigned>(count));

  // 1. moments (n times the covariances), regularised
  for (int32_t z = 0; z < count; ++z) {
    double* G = w.G + z * bs;
    double* C = w.C + z * bs;
    double* Gy = w.Gy + z * bs;
    double* sx = w.sx + z * bs;
    double* sy = w.sy + z * bs;
    if (int st = gram_one(x[z], ldx, y[z], ldy, in_f32, n_rows, f_in, f_out, w.part, G, C, s)) return st;
    if (int st = gram_one(y[z], ldy, y[z], ldy, in_f32, n_rows, f_out, 0, w.part, Gy, nullptr, s)) return st;
    if (int st = colsum(x[z], ldx, n_rows, f_in, in_f32, w.csp, sx, s)) return st;
    if (int st = colsum(y[z], ldy, n_rows, f_out, in_f32, w.csp, sy, s)) return st;
    center_kernel<<<grid_for(static_cast<int64_t>(f_in) * (f_in + f_out)), 256, 0, s>>>(G, C, sx, sy, f_in, f_out,
                                                                                        inv_n, 0);
    center_kernel<<<grid_for(fo2), 256, 0, s>>>(Gy, nullptr, sy, sy, f_out, 0, inv_n, 0);
    KVX_LAUNCH_CHECK();
    lambda_kernel<<<1, 256, 0, s>>>(G, f_in, 0.0, rho_x, w.lam + z * bs);
    lambda_kernel<<<1, 256, 0, s>>>(Gy, f_out, 0.0, rho_y, w.lam + z * bs + 1);
    KVX_LAUNCH_CHECK();
  }
  return recolor_solve(w, count, f_in, f_out, inv_n, w_out, b_out, status, iters, s);
}

// Steps 2-4 of the Recolor fit from the regularised moments in w (G, C, Gy,
// and the column sums sx, sy, n times the covariances; only G's lower
// triangle and diagonal tiles are read): every problem of the call at once.
static int recolor_solve(RcWs& w, int32_t count, int32_t f_in, int32_t f_out, double inv_n, float* const* w_out,
                         float* const* b_out, int32_t* status, int32_t* iters, hipStream_t s) {
  const int64_t bs = w.bs;
  const int64_t fo2 = static_cast<int64_t>(f_out) * f_out;
  const dim3 grid_o2(grid_for(fo2 / 8 + 1), static_cast<unsigned>(count));

  // 2. factors, Z0 = L_x^-1 C and E = L_y^-1 (the whitened cross-covariance
  // is M = Z0 E^T)
  if (int st = chol_factor(s, count, w.G, f_in, bs, w.linvx, w.xinvx, w.zbuf, w.flags)) return st;
  if (int st = chol_factor(s, count, w.Gy, f_out, bs, w.linvy, w.xinvy, w.zbuf, w.flags)) return st;
  zero_upper_kernel<<<grid_o2, 256, 0, s>>>(w.Gy, f_out, bs);
  KVX_LAUNCH_CHECK();
  if (int st = chol_forward(s, count, w.G, f_in, bs, w.xinvx, w.zbuf, w.C, f_out)) return st;
  identity_kernel<<<grid_o2, 256, 0, s>>>(w.E, f_out, bs);
  KVX_LAUNCH_CHECK();
  if (int st = chol_forward(s, count, w.Gy, f_out, bs, w.xinvy, w.zbuf, w.E, f_out)) return st;  // E = L_y^-1

  std::vector<int32_t> flags(static_cast<size_t>(count), 0);
  KVX_HIP_TRY(hipMemcpyAsync(flags.data(), w.flags, sizeof(int32_t) * count, hipMemcpyDeviceToHost, s));

  // 3. S = M^T M with M = Z0 E^T (Z0 = L_x^-1 S_xy, in C) formed as
  // E (Z0^T Z0) E^T, so the f_in x f_out matrix M is never formed (K in T,
  // E K in N, S in Y); then the polar iteration
  double *Y = w.ns[0], *Z = w.ns[1], *T = w.ns[2], *N = w.ns[3];
  // K, S and each step's T are symmetric (the iterates are polynomials in
  // S): only their tiles on and below the diagonal are formed, then mirrored.
  // Y and Z are updated by the full products with the one symmetric T, from
  // opposite sides: mirroring them as well breaks the pairing of their
  // rounding errors that keeps the coupled iteration stable (it then
  // diverges once Z grows large), so they stay as computed.
  if (int st = dgemm(s, count, f_out, f_out, f_in, w.C, 1, f_out, w.C, f_out, 1, T, f_out, bs, 1, 1)) return st;
  if (int st = sym_from_lower(s, count, T, f_out, bs)) return st;
  if (int st = dgemm(s, count, f_out, f_out, f_out, w.E, f_out, 1, T, f_out, 1, N, f_out, bs, 0, 1)) return st;
  if (int st = dgemm(s, count, f_out, f_out, f_out, N, f_out, 1, w.E, 1, f_out, Y, f_out, bs, 1, 1)) return st;
  if (int st = sym_from_lower(s, count, Y, f_out, bs)) return st;
  if (int st = frob(s, count, Y, f_out, bs, w.dev, w.scal)) return st;
  // largest eigenvalue of S by RC_POWER power steps (v in T, S v in N), so
  // the iteration starts with the spectrum of S / c close to (0, 1]: each
  // factor 2.25 of underscaling of the smallest eigenvalue costs one step
  power_start_kernel<<<static_cast<unsigned>(count), 256, 0, s>>>(T, f_out, bs);
  KVX_LAUNCH_CHECK();
  for (int it_p = 0; it_p < RC_POWER; ++it_p) {
    if (int st = dgemm(s, count, f_out, 1, f_out, Y, f_out, 1, T, 1, 1, N, 1, bs, 0, 1)) return st;
    power_norm_kernel<<<static_cast<unsigned>(count), 256, 0, s>>>(N, T, f_out, bs, w.scal + 2);
    KVX_LAUNCH_CHECK();
  }
  polar_scale_kernel<<<static_cast<unsigned>(count), 64, 0, s>>>(w.scal, bs);
  scale_kernel<<<grid_o2, 256, 0, s>>>(Y, fo2, bs, w.scal, -1.0);
  identity_kernel<<<grid_o2, 256, 0, s>>>(Z, f_out, bs);
  KVX_LAUNCH_CHECK();
  std::vector<double> dev(static_cast<size_t>(count) * NS_BLOCKS), prev(static_cast<size_t>(count), 1e300);
  std::vector<uint8_t> done(static_cast<size_t>(count), 0);
  int32_t it = 0;
  for (; it < RC_MAX_ITERS; ++it) {
    // third order: P = Z Y and P^2 (both symmetric), T = (15 I - 10 P + 3 P^2) / 8
    if (int st = dgemm(s, count, f_out, f_out, f_out, Z, f_out, 1, Y, f_out, 1, T, f_out, bs, 1, 1)) return st;
    if (int st = sym_from_lower(s, count, T, f_out, bs)) return st;
    if (int st = dgemm(s, count, f_out, f_out, f_out, T, f_out, 1, T, f_out, 1, N, f_out, bs, 1, 1)) return st;
    if (int st = sym_from_lower(s, count, N, f_out, bs)) return st;
    ns_mid_kernel<<<dim3(NS_BLOCKS, static_cast<unsigned>(count)), 256, 0, s>>>(T, N, f_out, bs, w.dev);
    KVX_LAUNCH_CHECK();
    if (int st = dgemm(s, count, f_out, f_out, f_out, Y, f_out, 1, T, f_out, 1, N, f_out, bs, 0, 1)) return st;
    std::swap(Y, N);
    if (int st = dgemm(s, count, f_out, f_out, f_out, T, f_out, 1, Z, f_out, 1, N, f_out, bs, 0, 1)) return st;
    std::swap(Z, N);
    KVX_HIP_TRY(hipMemcpyAsync(dev.data(), w.dev, sizeof(double) * dev.size(), hipMemcpyDeviceToHost, s));
    KVX_HIP_TRY(hipStreamSynchronize(s));
    bool all = true;
    for (int32_t z = 0; z < count; ++z) {
      if (flags[z] || done[z]) continue;
      double m = 0.0;
      for (int b = 0; b < NS_BLOCKS; ++b) m += dev[static_cast<size_t>(z) * NS_BLOCKS + b];
      m = std::sqrt(m);
      // converged with this step, at the rounding floor, or NaN (then Z is
      // NaN too and the problem reports that it did not converge)
      if (m <= RC_TOL || (m <= RC_FLOOR && m >= 0.25 * prev[z]) || m != m)
        done[z] = 1;
      else
        all = false;
      prev[z] = m;
    }
    if (all) {
      ++it;
      break;
    }
  }
  if (iters) *iters = it;
  if (int st = frob(s, count, Z, f_out, bs, w.dev, w.scal + 1)) return st;
  std::vector<double> zf(static_cast<size_t>(count));
  for (int32_t z = 0; z < count; ++z)
    KVX_HIP_TRY(hipMemcpyAsync(&zf[z], w.scal + z * bs + 1, sizeof(double), hipMemcpyDeviceToHost, s));

  // 4. W = L_x^-T Q L_y^T with Q = M S^-1/2 = Z0 E^T S^-1/2, S^-1/2 = Z / sqrt(c):
  // R = (E^T S^-1/2) L_y^T in the f_out x f_out products (Y, then T), then
  // W = L_x^-T (Z0 R); b = mean_y - mean_x W
  scale_kernel<<<grid_o2, 256, 0, s>>>(Z, fo2, bs, w.scal, -0.5);
  KVX_LAUNCH_CHECK();
  if (int st = dgemm(s, count, f_out, f_out, f_out, w.E, 1, f_out, Z, f_out, 1, Y, f_out, bs, 0, 1)) return st;
  if (int st = dgemm(s, count, f_out, f_out, f_out, Y, f_out, 1, w.Gy, 1, f_out, T, f_out, bs, 0, 1)) return st;
  if (int st = dgemm(s, count, f_in, f_out, f_out, w.C, f_out, 1, T, f_out, 1, w.M, f_out, bs, 0, 1)) return st;
  if (int st = chol_backward(s, count, w.G, f_in, bs, w.xinvx, w.zbuf, w.M, f_out)) return st;
  for (int32_t z = 0; z < count; ++z) {
    if (int st = fit_output(s, w.M + z * bs, f_in, f_out, w_out[z], b_out[z], w.sx + z * bs, w.sy + z * bs, inv_n,
                            w.csp))
      return st;
  }
  KVX_HIP_TRY(hipStreamSynchronize(s));
  int result = KVX_OK;
  for (int32_t z = 0; z < count; ++z) {
    const bool determined = done[z] && zf[z] <= RC_ZMAX;  // false for NaN too
    const int st = flags[z] ? KVX_ERR_NOT_SPD : (determined ? KVX_OK : KVX_ERR_NOT_CONVERGED);
    if (status) status[z] = st;
    if (st != KVX_OK && result == KVX_OK) result = st;
  }
  return result;
}

// Recolor fits of every receiver layer of n_roles roles from the
// calibration caches: the moments X^T X, X^T Y and the feature column sums
// from the alignment's runs (gram_from_runs), Y^T Y and the target column
// sums from each receiver layer's rows, then the solve of launch_recolor.
struct RccWs {
  RcWs rc;
  RunsWs r;
  uint16_t* ybuf;  // a receiver layer's keys rotated back, when they are stored rotated
  size_t bytes;
};

static RccWs recolor_caches_layout(const FitcShape& sh, void* base) {
  RccWs w{};
  w.rc = recolor_layout(sh.count, sh.f_in, sh.f_out, base);
  Carve c(base);
  c.used = w.rc.bytes;
  w.r = runs_layout(sh, c);
  if (sh.recv_rope > 0.0) w.ybuf = c.take<uint16_t>(static_cast<size_t>(sh.n_recv) * sh.f_out);
  w.bytes = c.used + 256;
  return w;
}

size_t recolor_caches_ws_bytes(const FitcShape& sh) { return recolor_caches_layout(sh, nullptr).bytes; }

int launch_recolor_caches(const FitcShape& sh, const void* const* send_role, const void* const* recv_role,
                          const int32_t* map, const int32_t* taps_host, double rho_x, double rho_y,
                          float* const* w_role, float* const* b_role, int32_t* status, int32_t* iters, void* ws,
                          hipStream_t s) {
  RccWs w = recolor_caches_layout(sh, ws);
  RcWs& rc = w.rc;
  const int64_t bs = rc.bs;
  if (int st = launch_fill_i32(rc.flags, sh.count, 0, s)) return st;
  if (int st = gram_from_runs(sh, w.r, send_role, recv_role, map, taps_host, rc.G, rc.C, rc.sx, bs, s)) return st;
  const double inv_n = 1.0 / static_cast<double>(sh.n_recv);
  const int64_t fo2 = static_cast<int64_t>(sh.f_out) * sh.f_out;
  // the targets' moments: Y^T Y of a role's layers in batched Gram launches,
  // the column sums per layer; target keys stored rotated are rotated back
  // one layer at a time first (the table was built for the run sums)
  const int64_t part_cap = static_cast<int64_t>(GR_MAX_SPLIT) * sh.f_in * (static_cast<int64_t>(sh.f_in) + sh.f_out);
  const int64_t y_layer = static_cast<int64_t>(sh.n_recv) * sh.f_out;
  for (int32_t r = 0; r < sh.n_roles; ++r) {
    const uint16_t* yr = static_cast<const uint16_t*>(recv_role[r]);
    const int64_t z0 = static_cast<int64_t>(r) * sh.recv_layers;
    const bool rot = r == sh.key_role && sh.recv_rope > 0.0;
    if (!rot) {
      if (int st = gram_batch(yr, sh.f_out, y_layer, yr, sh.f_out, y_layer, sh.n_recv, sh.f_out, 0, sh.recv_layers,
                              rc.part, part_cap, rc.Gy + z0 * bs, nullptr, bs, s))
        return st;
      // the Gram's partials are added up: their room holds the sums' chunks
      if (int st = colsum_batch(yr, sh.f_out, y_layer, sh.n_recv, sh.f_out, sh.recv_layers,
                                reinterpret_cast<double*>(rc.part), part_cap / 2, rc.sy + z0 * bs, bs, s))
        return st;
      continue;
    }
    for (int32_t l = 0; l < sh.recv_layers; ++l) {
      const uint16_t* y = yr + l * y_layer;
      const int64_t z = z0 + l;
      if (rot) {
        const unsigned gx =
            static_cast<unsigned>(std::min<int64_t>(ceil_div(y_layer / 16, 256), 4096));
        fitc_gather_kernel<true><<<dim3(gx, 1), 256, 0, s>>>(y, 0, sh.f_out, nullptr, nullptr, sh.n_recv, sh.n_recv,
                                                             w.ybuf, 0, w.r.tab_recv, sh.recv_hd);
        KVX_LAUNCH_CHECK();
        y = w.ybuf;
        if (int st = gram_one(y, sh.f_out, y, sh.f_out, 0, sh.n_recv, sh.f_out, 0, rc.part, rc.Gy + z * bs, nullptr,
                              s))
          return st;
      }
      if (int st = colsum(y, sh.f_out, sh.n_recv, sh.f_out, 0, rc.csp, rc.sy + z * bs, s)) return st;
    }
  }
  // centring and the regularisers of every problem at once
  center_kernel<<<dim3(grid_for(static_cast<int64_t>(sh.f_in) * (sh.f_in + sh.f_out)),
                       static_cast<unsigned>(sh.count)),
                  256, 0, s>>>(rc.G, rc.C, rc.sx, rc.sy, sh.f_in, sh.f_out, inv_n, bs);
  center_kernel<<<dim3(grid_for(fo2), static_cast<unsigned>(sh.count)), 256, 0, s>>>(rc.Gy, nullptr, rc.sy, rc.sy,
                                                                                    sh.f_out, 0, inv_n, bs);
  KVX_LAUNCH_CHECK();
  lambda_batched_kernel<<<static_cast<unsigned>(sh.count), 256, 0, s>>>(rc.G, bs, sh.f_in, 0.0, rho_x, rc.lam);
  lambda_batched_kernel<<<static_cast<unsigned>(sh.count), 256, 0, s>>>(rc.Gy, bs, sh.f_out, 0.0, rho_y, rc.lam + 1);
  KVX_LAUNCH_CHECK();
  std::vector<float*> w_out(static_cast<size_t>(sh.count)), b_out(static_cast<size_t>(sh.count));
  const int64_t nw = static_cast<int64_t>(sh.f_in) * sh.f_out;
  for (int32_t z = 0; z < sh.count; ++z) {
    w_out[z] = w_role[z / sh.recv_layers] + static_cast<int64_t>(z % sh.recv_layers) * nw;
    b_out[z] = b_role[z / sh.recv_layers] + static_cast<int64_t>(z % sh.recv_layers) * sh.f_out;
  }
  return recolor_solve(rc, sh.count, sh.f_in, sh.f_out, inv_n, w_out.data(), b_out.data(), status, iters, s);
}

}  // namespace kvx
