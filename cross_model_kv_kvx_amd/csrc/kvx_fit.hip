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
//      L^T W = Z by blocks;
//   4. W written output-major in fp32, b = mean_y - mean_x W.
// Several problems of one shape (the maps of every layer and role) are
// fitted by one call: steps 1, 2 and 4 run problem by problem (each fills
// the GPU), step 3 runs every launch of its serial chain over all problems
// at once, so the chain's latency is paid once per call.  A non-positive
// pivot sets the problem's device flag; the host reads the flags once.

#include <vector>

#include "kvx_internal.hpp"

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
  float* part;  // [split][f_in][f_in + f_out]
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
};

// Part of step k (64 rows) into `part`: load i of wave w covers part rows
// 2 (4w + i) and +1, lane j -> row + j/32, physical chunk j mod 32.  Steps
// past the end read nothing.
__device__ __forceinline__ void gr_issue(__amdgpu_buffer_rsrc_t r, uint32_t pitch, const uint32_t (&off)[GR_LD], int k,
                                         int nk, uint16_t* part) {
  const int wave = wave_id();
  const __amdgpu_buffer_rsrc_t rr = k < nk ? r : buf_rsrc(nullptr, 0);
  const uint32_t base = static_cast<uint32_t>(k) * GR_BK * pitch;
#pragma unroll
  for (int i = 0; i < GR_LD; ++i) dma16(rr, base + off[i], 0, part + (wave * GR_LD + i) * 512);
}

// One step: 4 x (2 P + 4 Q fragments, 8 MFMAs).
__device__ __forceinline__ void gr_compute(const uint16_t* pp, const uint16_t* pq, f32x16 (&acc)[2][4]) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;
  // lane of a 16-lane group g: the MFMA operand of lane l covers features
  // l mod 32 and rows 8 (l / 32) .. +7
  const int g = lane >> 4, s = lane & 15;
  const int r0 = 8 * (g >> 1) + (s >> 2);
  const int f0 = 16 * (g & 1) + 4 * (s & 3);
#pragma unroll
  for (int kk = 0; kk < GR_BK / 16; ++kk) {
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
  gr_issue(it.pr, it.p_pitch, it.p_off, (K) + 2, it.nk, NA); \
  if (LIVE) gr_compute(PA, PB, acc);

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
  const int64_t T = static_cast<int64_t>(g.split) * per;
  const int32_t G = gridDim.x;
  // consecutive items go to the workgroups of one XCD (dispatch is round
  // robin over the 8 XCDs)
  const int32_t slot = (G % 8 == 0) ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int64_t ldp = static_cast<int64_t>(g.f_in) + g.f_out;

  for (int64_t t = slot; t < T; t += G) {
    const int32_t sidx = static_cast<int32_t>(t / per);
    int32_t tt = static_cast<int32_t>(t % per);
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
    const uint16_t* q = is_c ? g.y : g.x;
    const int64_t ldq = is_c ? g.ldy : g.ldx;
    const int32_t fq = is_c ? g.f_out : g.f_in;

    GrItem it;
    it.p_pitch = static_cast<uint32_t>(2 * g.ldx);
    it.q_pitch = static_cast<uint32_t>(2 * ldq);
    // the range ends with the split's last row (features past the row's end
    // come from the next row and only reach outputs that are not written)
    it.pr = buf_rsrc(g.x + k_begin * g.ldx + i0, static_cast<uint32_t>(rows * 2 * g.ldx - 2 * i0));
    it.qr = buf_rsrc(q + k_begin * ldq + j0, static_cast<uint32_t>(rows * 2 * ldq - 2 * j0));
    if (rows == 0) {
      it.pr = buf_rsrc(nullptr, 0);
      it.qr = buf_rsrc(nullptr, 0);
    }
    it.nk = static_cast<int32_t>((rows + GR_BK - 1) / GR_BK);
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
      for (int k = 0; k < it.nk; k += 5) {
        GR_STEP(k, p0, p1, p3, p4, true)
        GR_STEP(k + 1, p2, p3, p0, p1, k + 1 < it.nk)
        GR_STEP(k + 2, p4, p0, p2, p3, k + 2 < it.nk)
        GR_STEP(k + 3, p1, p2, p4, p0, k + 3 < it.nk)
        GR_STEP(k + 4, p3, p4, p1, p2, k + 4 < it.nk)
      }
      KVX_WAIT_VM(0);
    }

    float* part = g.part + static_cast<int64_t>(sidx) * g.f_in * ldp + (is_c ? g.f_in : 0);
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
#undef GR_STEP

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

// Column sums of X and Y in fp64 (for the intercept).
template <bool F32>
__global__ __launch_bounds__(256) void colsum_kernel(const void* __restrict__ m, int64_t ld, int64_t n_rows,
                                                     int32_t cols, double* __restrict__ out) {
  const int32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  double s = 0.0;
  for (int64_t k = 0; k < n_rows; ++k)
    s += F32 ? static_cast<double>(static_cast<const float*>(m)[k * ld + c])
             : static_cast<double>(bf16_to_f32(static_cast<const uint16_t*>(m)[k * ld + c]));
  out[c] = s;
}

// Sum of the split partials in fp64 by 64 x 64 blocks of [G | C]: blocks of
// G on and above the diagonal and every block of C are read row by row
// (256-byte rows of each split); a block of G above the diagonal is also
// written to its mirror through an LDS transpose, so every global access
// walks rows.
constexpr int RD_T = 64;
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ part, int32_t split,
                                                          int32_t f_in, int32_t f_out, double* __restrict__ G,
                                                          double* __restrict__ C) {
  __shared__ double tr[RD_T][RD_T + 1];
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

// Centring: G -= sx sx^T / n, C -= sx sy^T / n.
__global__ __launch_bounds__(256) void center_kernel(double* __restrict__ G, double* __restrict__ C,
                                                     const double* __restrict__ sx, const double* __restrict__ sy,
                                                     int32_t f_in, int32_t f_out, double inv_n) {
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

// Factor the diagonal block [k0, k0+nb) (lower) of one problem of a batch
// (one workgroup per problem), flag non-positive pivots,
// and write the inverse of the factor (lower, nb x nb, zero above the
// diagonal, row stride CH_NB) to `linv`: the panel and the block triangular
// solves then become products with it.  One wave, no barrier: lane i keeps
// row i in registers; at column j every lane takes the pivot from lane j
// (the square root is recomputed per lane), lane i scales its entry and
// publishes it in LDS, and each lane updates its row with the published
// column (LDS operations of one wave execute in order).  Rows past nb are
// the identity.  The inverse is formed one column per lane by forward
// substitution against the factor in LDS.
__global__ __launch_bounds__(64) void potrf_diag_kernel(double* __restrict__ A, int64_t bsa, int32_t n, int32_t k0,
                                                        int32_t nb, int32_t* __restrict__ flag,
                                                        double* __restrict__ linv, int64_t bsl) {
  // problem blockIdx.x of a batch
  A += blockIdx.x * bsa;
  flag += blockIdx.x;
  linv += blockIdx.x * bsl;
  __shared__ double L[CH_NB][CH_NB + 1];
  __shared__ double col[CH_NB];
  const int i = threadIdx.x;
  double row[CH_NB];
#pragma unroll
  for (int c = 0; c < CH_NB; ++c)
    row[c] = (i < nb && c < nb) ? A[static_cast<int64_t>(k0 + i) * n + k0 + c] : (i == c ? 1.0 : 0.0);
  int bad = 0;
#pragma unroll
  for (int j = 0; j < CH_NB; ++j) {
    // pivot of column j, from lane j
    const double d = __shfl(row[j], j, 64);
    const bool ok = d > 0.0;
    if (j < nb && !ok) bad = 1;
    const double piv = sqrt(ok ? d : 1.0);
    const double rp = 1.0 / piv;
    if (i == j) row[j] = piv;
    if (i > j) row[j] *= rp;
    col[i] = row[j];
    KVX_COMPILER_FENCE();
#pragma unroll
    for (int c = j + 1; c < CH_NB; ++c) {
      const double lc = col[c];
      if (i >= c) row[c] -= row[j] * lc;
    }
    KVX_COMPILER_FENCE();
  }
  if (bad && i == 0) *flag = 1;
#pragma unroll
  for (int c = 0; c < CH_NB; ++c) L[i][c] = (c <= i) ? row[c] : 0.0;
  KVX_COMPILER_FENCE();
  // inverse: lane c forms column c
  double x[CH_NB];
  const int c = i;
#pragma unroll
  for (int r = 0; r < CH_NB; ++r) {
    double v = (r == c) ? 1.0 : 0.0;
#pragma unroll
    for (int q = 0; q < r; ++q) v -= L[r][q] * x[q];
    x[r] = (r >= c) ? v / L[r][r] : 0.0;
  }
#pragma unroll
  for (int r = 0; r < CH_NB; ++r) {
    if (i < nb && r < nb && r >= i) A[static_cast<int64_t>(k0 + r) * n + k0 + i] = L[r][i];
    linv[r * CH_NB + c] = (r < nb && c < nb) ? x[r] : 0.0;
  }
}

// C[M x N] -= A * B (overwrite = 0) or C = A * B (overwrite = 1) in fp64 on
// matrix cores, for a batch of problems (blockIdx.z; the operands of problem
// z start bsa, bsb, bsc elements after those of problem z-1), with
// A(m,k) = A[m*sam + k*sak] and B(k,n) = B[k*sbk + n*sbn].  64 x 64 tiles;
// four waves of 32 x 32, each from 2 x 2 MFMA 16x16x4 fp64 blocks; K in steps
// of 16 through LDS as [k][m] and [k][n] (global elements are read along the
// operand's unit-stride index; rows padded so the 16-lane row pieces of a
// fragment read fall in distinct banks).  A workgroup reads all of its A rows
// and B columns before it writes its tile, so C may alias A when N <= 64 or B
// when M <= 64.  lower_only skips tiles strictly above the diagonal.
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
constexpr int DG_T = 64;
constexpr int DG_BK = 16;
constexpr int DG_LD = DG_T + 16;

// The next K chunk is read into registers while the current one is
// multiplied, and an updated C tile is read before the K loop, so both
// latencies overlap the matrix instructions.
__global__ __launch_bounds__(256) void dgemm_kernel(const DgArgs g) {
  const int32_t bm = blockIdx.y, bn = blockIdx.x;
  if (g.lower_only && bm < bn) return;
  __shared__ double As[DG_BK][DG_LD];
  __shared__ double Bs[DG_BK][DG_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int32_t m0 = bm * DG_T, n0 = bn * DG_T;
  const double* A = g.A + blockIdx.z * g.bsa;
  const double* B = g.B + blockIdx.z * g.bsb;
  double* C = g.C + blockIdx.z * g.bsc;
  const bool a_k = g.sak == 1 && g.sam != 1;  // A read along k
  const bool b_k = g.sbk == 1 && g.sbn != 1;  // B read along k

  double av[4], bv[4];
  auto load = [&](int32_t k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int ma = a_k ? (e >> 4) : (e & 63), ka = a_k ? (e & 15) : (e >> 6);
      const int32_t m = m0 + ma, k = k0 + ka;
      av[q] = (m < g.M && k < g.K) ? A[m * g.sam + k * g.sak] : 0.0;
      const int nb_ = b_k ? (e >> 4) : (e & 63), kb = b_k ? (e & 15) : (e >> 6);
      const int32_t n = n0 + nb_, kq = k0 + kb;
      bv[q] = (n < g.N && kq < g.K) ? B[kq * g.sbk + n * g.sbn] : 0.0;
    }
  };
  // element r of lane l: row l/16 + 4r, column l%16 of its 16 x 16 block
  auto row_of = [&](int i, int r) { return m0 + wm * 32 + i * 16 + (lane >> 4) + 4 * r; };
  auto col_of = [&](int j) { return n0 + wn * 32 + j * 16 + (lane & 15); };

  f64x4 acc[2][2], cv[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
      cv[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
    }
  load(0);
  if (!g.overwrite) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t m = row_of(i, r), n = col_of(j);
          if (m < g.M && n < g.N) cv[i][j][r] = C[m * g.ldc + n];
        }
  }
  for (int32_t k0 = 0; k0 < g.K; k0 += DG_BK) {
    __syncthreads();  // the previous chunk's fragment reads are done
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      As[a_k ? (e & 15) : (e >> 6)][a_k ? (e >> 4) : (e & 63)] = av[q];
      Bs[b_k ? (e & 15) : (e >> 6)][b_k ? (e >> 4) : (e & 63)] = bv[q];
    }
    __syncthreads();
    if (k0 + DG_BK < g.K) load(k0 + DG_BK);
#pragma unroll
    for (int k4 = 0; k4 < DG_BK; k4 += 4) {
      // operands of MFMA 16x16x4: lane l holds A[l%16][l/16] and B[l/16][l%16]
      const int kr = k4 + (lane >> 4);
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[kr][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[kr][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int32_t m = row_of(i, r), n = col_of(j);
        if (m < g.M && n < g.N) C[m * g.ldc + n] = g.overwrite ? acc[i][j][r] : cv[i][j][r] - acc[i][j][r];
      }
}

// w_out[o][f] = W[f][o] (fp32); b_out[o] = mean_y[o] - sum_f mean_x[f] W[f][o].
__global__ __launch_bounds__(256) void fit_output_kernel(const double* __restrict__ W, int32_t f_in, int32_t f_out,
                                                         float* __restrict__ w_out, float* __restrict__ b_out,
                                                         const double* __restrict__ sx, const double* __restrict__ sy,
                                                         double inv_n) {
  const int64_t total = static_cast<int64_t>(f_in) * f_out;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int32_t o = static_cast<int32_t>(e / f_in), f = static_cast<int32_t>(e % f_in);
    w_out[e] = static_cast<float>(W[static_cast<int64_t>(f) * f_out + o]);
  }
  if (b_out) {
    for (int32_t o = blockIdx.x * blockDim.x + threadIdx.x; o < f_out; o += gridDim.x * blockDim.x) {
      double s = sy[o] * inv_n;
      for (int32_t f = 0; f < f_in; ++f) s -= sx[f] * inv_n * W[static_cast<int64_t>(f) * f_out + o];
      b_out[o] = static_cast<float>(s);
    }
  }
}

// ---------------------------------------------------------------- host side

// Workspace: the Gram partials (shared by the problems, which are
// accumulated one after the other), then per problem G, C, column sums,
// lambda and the inverse diagonal factors, then one flag per problem.
struct FitWs {
  float* part;
  double *G, *C, *sx, *sy, *lam, *linv;
  int64_t bs;  // doubles between the per-problem areas
  int64_t oG, oC, oSx, oSy, oLam, oLinv;
  int32_t* flags;
  size_t bytes;
};

static FitWs fit_layout(int32_t count, int32_t f_in, int32_t f_out, void* base) {
  FitWs w{};
  Carve c(base);
  w.part = c.take<float>(static_cast<size_t>(GR_MAX_SPLIT) * f_in * (static_cast<size_t>(f_in) + f_out));
  const int64_t nb_total = ceil_div(f_in, CH_NB);
  auto up = [](int64_t v) { return (v + 31) / 32 * 32; };  // 256-byte sub-areas
  w.oG = 0;
  w.oC = w.oG + up(static_cast<int64_t>(f_in) * f_in);
  w.oSx = w.oC + up(static_cast<int64_t>(f_in) * f_out);
  w.oSy = w.oSx + up(f_in);
  w.oLam = w.oSy + up(f_out);
  w.oLinv = w.oLam + up(4);
  w.bs = w.oLinv + up(nb_total * CH_NB * CH_NB);
  double* area = c.take<double>(static_cast<size_t>(count) * w.bs);
  if (area) {
    w.G = area + w.oG;
    w.C = area + w.oC;
    w.sx = area + w.oSx;
    w.sy = area + w.oSy;
    w.lam = area + w.oLam;
    w.linv = area + w.oLinv;
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
  const dim3 grid(static_cast<unsigned>(ceil_div(N, DG_T)), static_cast<unsigned>(ceil_div(M, DG_T)),
                  static_cast<unsigned>(count));
  dgemm_kernel<<<grid, 256, 0, s>>>(g);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// Gram and cross products of one problem into its G and C.
static int gram_one(const void* x, int64_t ldx, const void* y, int64_t ldy, int32_t in_f32, int64_t n_rows,
                    int32_t f_in, int32_t f_out, float* part, double* G, double* C, hipStream_t s) {
  if (in_f32) {
    gram_f32_kernel<<<grid_for(static_cast<int64_t>(f_in) * (f_in + f_out)), 256, 0, s>>>(
        static_cast<const float*>(x), ldx, static_cast<const float*>(y), ldy, n_rows, f_in, f_out, G, C);
    KVX_LAUNCH_CHECK();
    return KVX_OK;
  }
  GramArgs g{};
  g.x = static_cast<const uint16_t*>(x);
  g.y = static_cast<const uint16_t*>(y);
  g.ldx = ldx;
  g.ldy = ldy;
  g.n_rows = n_rows;
  g.f_in = f_in;
  g.f_out = f_out;
  g.nbi = static_cast<int32_t>(ceil_div(f_in, GR_T));
  g.nbc = static_cast<int32_t>(ceil_div(f_out, GR_T));
  g.n_g = g.nbi * (g.nbi + 1) / 2;
  g.n_c = g.nbi * g.nbc;
  // row splits: the fewest that fill the persistent grid best (fewer
  // partials to add up, longer K loops), each at least one step long
  const int cus = device_cu_count();
  const int64_t tiles = g.n_g + g.n_c;
  int64_t split = 1;
  double best = 0.0;
  for (int64_t sp = 1; sp <= GR_MAX_SPLIT; ++sp) {
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
  {
    const int64_t nbi = ceil_div(f_in, RD_T), nbc = ceil_div(f_out, RD_T);
    gram_reduce_kernel<<<static_cast<unsigned>(nbi * (nbi + 1) / 2 + nbi * nbc), 256, 0, s>>>(part, g.split, f_in,
                                                                                               f_out, G, C);
  }
  KVX_LAUNCH_CHECK();
  return KVX_OK;
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
      if (in_f32) {
        colsum_kernel<true><<<grid_for(f_in), 256, 0, s>>>(x[z], ldx, n_rows, f_in, sx);
        colsum_kernel<true><<<grid_for(f_out), 256, 0, s>>>(y[z], ldy, n_rows, f_out, sy);
      } else {
        colsum_kernel<false><<<grid_for(f_in), 256, 0, s>>>(x[z], ldx, n_rows, f_in, sx);
        colsum_kernel<false><<<grid_for(f_out), 256, 0, s>>>(y[z], ldy, n_rows, f_out, sy);
      }
      KVX_LAUNCH_CHECK();
      center_kernel<<<grid_for(static_cast<int64_t>(f_in) * (f_in + f_out)), 256, 0, s>>>(G, C, sx, sy, f_in, f_out,
                                                                                          inv_n);
      KVX_LAUNCH_CHECK();
    }
    lambda_kernel<<<1, 256, 0, s>>>(G, f_in, lam_abs, lam_rel, w.lam + z * bs);
    KVX_LAUNCH_CHECK();
  }

  // 2. Cholesky and the two block triangular solves of all problems at once;
  // the diagonal kernel leaves the inverse factor of its block, so each panel
  // and each block solve is an in-place product with it.
  const int32_t nb_total = static_cast<int32_t>(ceil_div(f_in, CH_NB));
  for (int32_t kb = 0; kb < nb_total; ++kb) {
    const int32_t k0 = kb * CH_NB;
    const int32_t nb = min(CH_NB, f_in - k0);
    double* li = w.linv + static_cast<int64_t>(kb) * CH_NB * CH_NB;
    potrf_diag_kernel<<<static_cast<unsigned>(count), 64, 0, s>>>(w.G, bs, f_in, k0, nb, w.flags, li, bs);
    KVX_LAUNCH_CHECK();
    const int32_t rest = f_in - k0 - nb;
    if (rest > 0) {
      // panel: P = P L_kk^-T (in place, one 64-column tile)
      double* P = w.G + static_cast<int64_t>(k0 + nb) * f_in + k0;
      if (int st = dgemm(s, count, rest, nb, nb, P, f_in, 1, li, 1, CH_NB, P, f_in, bs, 0, 1)) return st;
      // trailing lower update: G[r][c] -= P[r] . P[c] for r, c >= k0+nb
      double* Ct = w.G + static_cast<int64_t>(k0 + nb) * f_in + k0 + nb;
      if (int st = dgemm(s, count, rest, rest, nb, P, f_in, 1, P, 1, f_in, Ct, f_in, bs, 1, 0)) return st;
    }
  }
  // forward: L Z = C
  for (int32_t kb = 0; kb < nb_total; ++kb) {
    const int32_t k0 = kb * CH_NB;
    const int32_t nb = min(CH_NB, f_in - k0);
    const double* li = w.linv + static_cast<int64_t>(kb) * CH_NB * CH_NB;
    double* Zk = w.C + static_cast<int64_t>(k0) * f_out;
    // Z_k = L_kk^-1 Z_k (in place, one 64-row tile)
    if (int st = dgemm(s, count, nb, f_out, nb, li, CH_NB, 1, Zk, f_out, 1, Zk, f_out, bs, 0, 1)) return st;
    const int32_t rest = f_in - k0 - nb;
    if (rest > 0) {
      const double* Lb = w.G + static_cast<int64_t>(k0 + nb) * f_in + k0;
      double* Cr = w.C + static_cast<int64_t>(k0 + nb) * f_out;
      if (int st = dgemm(s, count, rest, f_out, nb, Lb, f_in, 1, Zk, f_out, 1, Cr, f_out, bs, 0, 0)) return st;
    }
  }
  // backward: L^T W = Z
  for (int32_t kb = nb_total - 1; kb >= 0; --kb) {
    const int32_t k0 = kb * CH_NB;
    const int32_t nb = min(CH_NB, f_in - k0);
    const double* li = w.linv + static_cast<int64_t>(kb) * CH_NB * CH_NB;
    double* Wk = w.C + static_cast<int64_t>(k0) * f_out;
    // W_k = L_kk^-T W_k (in place)
    if (int st = dgemm(s, count, nb, f_out, nb, li, 1, CH_NB, Wk, f_out, 1, Wk, f_out, bs, 0, 1)) return st;
    if (k0 > 0) {
      // Z[0..k0) -= L[k0..k0+nb)[0..k0)^T W_k
      const double* Lr = w.G + static_cast<int64_t>(k0) * f_in;
      if (int st = dgemm(s, count, k0, f_out, nb, Lr, 1, f_in, Wk, f_out, 1, w.C, f_out, bs, 0, 0)) return st;
    }
  }

  // 3. outputs
  for (int32_t z = 0; z < count; ++z) {
    fit_output_kernel<<<grid_for(static_cast<int64_t>(f_in) * f_out), 256, 0, s>>>(
        w.C + z * bs, f_in, f_out, w_out[z], fit_intercept ? b_out[z] : nullptr, w.sx + z * bs, w.sy + z * bs,
        inv_n);
    KVX_LAUNCH_CHECK();
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

}  // namespace kvx
