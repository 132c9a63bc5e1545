// Flattened cross-head translation on matrix cores.
//
// "Prefill-Free Cross-Family KV Cache Transfer ..." (Methodology 2): each
// receiver layer reads three sender layers (matched layer and its -4/+4
// neighbours), concatenates their whole rows (all heads) and maps them with
// one affine map per layer and role, so head counts need not agree.  With
// token alignment many receiver tokens reuse one sender token, so the product
// is formed once per run of equal sender indices (U distinct rows) and the
// epilogue writes it to every receiver row of the run, rotating keys at each
// receiver position ("Cross-Model KV Cache Transfer in Production", stage 4).
//
// One launch is a persistent grouped GEMM over (role, receiver layer)
// problems, each T[U x F_out] = A[U x K] * W^T + b, with 16-bit operands of
// one type per role (bf16, or fp16 for rotated-back keys) and fp32
// accumulation:
//   * block tile 256 (rows) x 256 (outputs = two 128-wide heads), 4 waves of
//     128 x 128, each built from 4 x 4 MFMA 32x32x16 accumulators;
//   * K advances 32 elements per step through a ring of 4 LDS stages (32 KB
//     each) filled by direct global->LDS 16-byte loads: A rows are gathered
//     per lane (sender token of each run, or a compact rotated-back row) and
//     W rows are read output-major, so no staging registers are needed and
//     three steps stay in flight while one is multiplied;
//   * 16-byte chunks are XOR-swizzled inside each 64-byte LDS row so the
//     fragment reads of 16 consecutive rows hit distinct banks;
//   * each stage is a separate LDS array so the compiler can keep counted
//     vmcnt waits (a single array would force a full drain before every LDS
//     read), and the only synchronisation per step is one s_barrier;
//   * tiles of one problem are grouped 8 (rows) x F_out/256 (outputs) and one
//     group goes to the 32 blocks of one XCD (blocks are dispatched round
//     robin over the 8 XCDs), so A and W slices are shared in that XCD's L2;
//   * epilogue: each wave stages 64 rows x 128 outputs (bias added) in its
//     own ring slot, then walks the receiver rows of those runs 8 at a time,
//     rotating key pairs (c, c+64) at the receiver position by a recurrence
//     and storing 2 x 16 bytes of bf16 (nearest even) per lane.

#include "kvx_internal.hpp"

namespace kvx {

constexpr int FT_M = 256;
constexpr int FT_N = 256;
constexpr int FT_BK = 32;
constexpr int FT_THREADS = 256;
constexpr int FT_SLOT_ELEMS = (FT_M + FT_N) * FT_BK;  // 16-bit elements per stage (32 KB)
constexpr int FT_B_OFF = FT_M * FT_BK;                // B tile offset inside a stage

struct FlatKArgs {
  const uint16_t* a_src[2];
  int64_t a_layer_stride[2];
  int32_t a_compact[2];
  int32_t a_f16[2];
  const uint16_t* wt[2];  // [L_R][F_out][K], K = k_dim
  const float* bias[2];
  uint16_t* out[2];
  int32_t rotate[2];
  int32_t n_roles;
  int32_t recv_layers, recv_tokens, k_dim, f_out, send_row, n_taps;
  const float2* tab_recv;
  const int32_t* uniq;
  const int32_t* run_begin;
  const int32_t* r2u;
  const int32_t* n_uniq;
  // taps of layer l: bytes of taps[l][0] (taps 0..3) and taps[l][1] (4..6);
  // dword-packed so they are read with scalar loads
  uint32_t taps[MAX_LAYERS][2];
};

typedef __attribute__((address_space(3))) void lds_void_t;

// Buffer resource over [base, base + bytes) for raw 32-bit loads (word 3 as
// for gfx9 raw buffers); loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ft_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// 16 bytes per lane from the buffer at voffset + soffset (per-lane and
// uniform byte offsets) into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds), 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(N) leaving the other counters unconstrained (gfx9 encoding:
// vmcnt[3:0] bits 3:0, expcnt bits 6:4, lgkmcnt bits 11:8, vmcnt[5:4] bits 15:14).
#define FT_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | 0x70 | 0xF00)
#define FT_COMPILER_FENCE() asm volatile("" ::: "memory")

// Two fp32 -> packed bf16 (hardware convert, round to nearest even).
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Per-tile addressing of this thread's direct loads.  Load instruction i of
// wave w covers tile rows (4w + i) * 16 .. +16; lane j lands at row +j/4,
// physical chunk j%4, and fetches logical chunk (j%4) ^ ((j/16)%4).
struct TileAddr {
  const char* a_src;            // A source, layer 0
  int64_t a_ls;                 // bytes between A source layers (< 2^31)
  uint32_t taps0, taps1;        // sender layer of taps 0..3 and 4..6, one byte each
  __amdgpu_buffer_rsrc_t w_r;   // map rows n0 .. n0+255 of this layer
  uint32_t a_off[4];            // byte offsets of the A rows (row * send_row + chunk)
  uint32_t b_off[4];            // byte offsets of the W rows
  int32_t spt;                  // K steps per tap (send_row / 32)
  int32_t n_taps;
};

// Wave index as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ void ft_issue(const TileAddr& ta, int k, uint16_t* slot) {
  const int wave = wave_id();
  const int32_t tap_i = k / ta.spt;
  const int32_t w0 = (k - tap_i * ta.spt) * FT_BK;
  const int32_t tap = tap_i % ta.n_taps;  // fp32 maps split in two repeat the taps
  const uint32_t layer = ((tap < 4 ? ta.taps0 : ta.taps1) >> (8 * (tap & 3))) & 0xffu;
  const __amdgpu_buffer_rsrc_t a_r = ft_rsrc(ta.a_src + static_cast<int64_t>(layer) * ta.a_ls,
                                             static_cast<uint32_t>(ta.a_ls));
  const uint32_t a_soff = 2u * static_cast<uint32_t>(w0);
  const uint32_t b_soff = 2u * static_cast<uint32_t>(k * FT_BK);
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16(a_r, ta.a_off[i], a_soff, slot + (wave * 4 + i) * 512);
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16(ta.w_r, ta.b_off[i], b_soff, slot + FT_B_OFF + (wave * 4 + i) * 512);
}

// One K step from a stage: 2 x (4 A + 4 B fragment reads, 16 MFMAs).
template <bool F16>
__device__ __forceinline__ void ft_compute(const uint16_t* slot, f32x16 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave & 1, wn = wave >> 1;
  const char* sb = reinterpret_cast<const char*>(slot);
  const int fr = lane & 31;
  const int sw = (lane >> 2) & 3;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int pc = ((2 * kk + (lane >> 5)) ^ sw) << 4;
    u32x4 af[4], bfr[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) af[mi] = *reinterpret_cast<const u32x4*>(sb + (wm * 128 + mi * 32 + fr) * 64 + pc);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      bfr[ni] = *reinterpret_cast<const u32x4*>(sb + FT_B_OFF * 2 + (wn * 128 + ni * 32 + fr) * 64 + pc);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma32<F16>(af[mi], bfr[ni], acc[mi][ni]);
  }
}

// Wait until step k's loads have landed with `after` younger steps still in
// flight, then one barrier.
template <int AFTER>
__device__ __forceinline__ void ft_sync() {
  FT_WAIT_VM(8 * AFTER);
  FT_COMPILER_FENCE();
  __builtin_amdgcn_s_barrier();
  FT_COMPILER_FENCE();
}

// K loop over nk steps (nk a multiple of 4, >= 4) with steps 0..2 already
// issued into slots 0..2.  The main loop issues unconditionally (a
// conditional issue makes the compiler drain every load before LDS reads);
// the last four steps are peeled.
template <bool F16>
__device__ __forceinline__ void ft_kloop(const TileAddr& ta, int nk, uint16_t* s0, uint16_t* s1, uint16_t* s2,
                                         uint16_t* s3, f32x16 (&acc)[4][4]) {
  for (int k = 0; k < nk - 4; k += 4) {
    ft_sync<2>();
    ft_issue(ta, k + 3, s3);
    ft_compute<F16>(s0, acc);
    ft_sync<2>();
    ft_issue(ta, k + 4, s0);
    ft_compute<F16>(s1, acc);
    ft_sync<2>();
    ft_issue(ta, k + 5, s1);
    ft_compute<F16>(s2, acc);
    ft_sync<2>();
    ft_issue(ta, k + 6, s2);
    ft_compute<F16>(s3, acc);
  }
  ft_sync<2>();
  ft_issue(ta, nk - 1, s3);
  ft_compute<F16>(s0, acc);
  ft_sync<2>();
  ft_compute<F16>(s1, acc);
  ft_sync<1>();
  ft_compute<F16>(s2, acc);
  ft_sync<0>();
  ft_compute<F16>(s3, acc);
}

// F16: operand type of every role of this launch (fp16 or bf16).
template <bool F16>
__global__ __launch_bounds__(FT_THREADS, 1) void flat_gemm_kernel(const FlatKArgs args) {
  __shared__ __attribute__((aligned(1024))) uint16_t s0[FT_SLOT_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t s1[FT_SLOT_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t s2[FT_SLOT_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t s3[FT_SLOT_ELEMS];

  const int32_t U = *args.n_uniq;
  if (U <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = wave & 1, wn = wave >> 1;
  const int32_t mt = (U + FT_M - 1) / FT_M;
  const int32_t nt = args.f_out / FT_N;
  const int64_t per_p = static_cast<int64_t>(mt) * nt;
  const int64_t T = static_cast<int64_t>(args.n_roles) * args.recv_layers * per_p;
  const int32_t G = gridDim.x;
  const int32_t slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int32_t nk = args.k_dim / FT_BK;
  const int lrow = lane >> 2;                               // row inside a 16-row load group
  const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);        // logical chunk fetched by this lane

  for (int64_t t = slot; t < T; t += G) {
    const int32_t p = static_cast<int32_t>(t / per_p);
    const int32_t rr = static_cast<int32_t>(t % per_p);
    const int32_t mg = rr / (8 * nt);
    const int32_t r2 = rr % (8 * nt);
    const int32_t gm = min(8, mt - mg * 8);
    const int32_t n0 = (r2 / gm) * FT_N;
    const int32_t m0 = (mg * 8 + r2 % gm) * FT_M;
    const int role = p / args.recv_layers;
    const int l = p % args.recv_layers;

    TileAddr ta;
    ta.a_src = reinterpret_cast<const char*>(args.a_src[role]);
    ta.a_ls = 2 * args.a_layer_stride[role];
    ta.taps0 = args.taps[l][0];
    ta.taps1 = args.taps[l][1];
    ta.spt = args.send_row / FT_BK;
    ta.n_taps = args.n_taps;
    ta.w_r = ft_rsrc(reinterpret_cast<const char*>(args.wt[role] + (static_cast<int64_t>(l) * args.f_out + n0) * args.k_dim),
                     static_cast<uint32_t>(2 * FT_N * args.k_dim));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (wave * 4 + i) * 16 + lrow;
      int32_t u = m0 + r;
      u = u < U ? u : U - 1;
      const int32_t srow = args.a_compact[role] ? u : args.uniq[u];
      ta.a_off[i] = 2u * static_cast<uint32_t>(srow * args.send_row + lchunk * 8);
      ta.b_off[i] = 2u * static_cast<uint32_t>(r * args.k_dim + lchunk * 8);
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // prologue: steps 0..2 in flight.  Slots 0..2 were last read before the
    // final barrier of the previous tile, so they are free.
    ft_issue(ta, 0, s0);
    ft_issue(ta, 1, s1);
    ft_issue(ta, 2, s2);
    ft_kloop<F16>(ta, nk, s0, s1, s2, s3, acc);

    // ------------------------------------------------------------ epilogue
    // Each wave owns 128 unique rows x one 128-wide head, written in two
    // phases of 64 unique rows staged (bias added, fp32) in the wave's own
    // ring slot.  The phase's receiver rows P0 .. P1-1 are walked by 8 lane
    // groups, group g taking rows P0 + g + 8i (balanced, no divergence); lane
    // q of a group owns pairs 8q .. 8q+7.  The unique row of a receiver row
    // comes from the run index array (coalesced loads one round of 64 rows
    // ahead, distributed by shuffles).  Keys are rotated with a recurrence
    // stepping 8 positions, (cos, sin)((p+8)t) = (cos, sin)(pt) x
    // (cos, sin)(8t), started from the fp64-derived table once per phase.
    const int q = lane & 7;
    const int grp = lane >> 3;
    const int col = wn * 128 + 8 * q;  // tile column of the first pair member
    const float* bias = args.bias[role];
    float bcol[4];  // bias of the columns this lane stages (ni * 32 + lane % 32)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      bcol[ni] = bias ? bias[static_cast<int64_t>(l) * args.f_out + n0 + wn * 128 + ni * 32 + (lane & 31)] : 0.0f;
    const bool rot = args.rotate[role] != 0;
    uint16_t* outp = args.out[role] + static_cast<int64_t>(l) * args.recv_tokens * args.f_out + n0 + col;
    float* ep = reinterpret_cast<float*>(wave == 0 ? s0 : (wave == 1 ? s1 : (wave == 2 ? s2 : s3)));
    // every wave has finished reading the ring (the last step read slot 3)
    FT_COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    FT_COMPILER_FENCE();
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      const int32_t u0 = m0 + wm * 128 + 64 * ph;
      // stage rows 64*ph .. +64 (columns XOR 32 on rows with bit 2 set so the
      // two half-waves hit different banks); the scheduling barrier keeps the
      // accumulator reads of a phase here
      __builtin_amdgcn_sched_barrier(0);
      FT_COMPILER_FENCE();
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 32 * m2 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int cc = (ni * 32 + (lane & 31)) ^ (((row >> 2) & 1) << 5);
            ep[row * 128 + cc] = acc[2 * ph + m2][ni][r] + bcol[ni];
          }
      FT_COMPILER_FENCE();  // LDS operations of one wave execute in order
      __builtin_amdgcn_sched_barrier(0);
      if (u0 >= U) continue;
      const int32_t p0 = args.run_begin[u0];
      const int32_t n = args.run_begin[min(u0 + 64, U)] - p0;
      float cs[8], sn[8], c8[8], s8[8];
      if (rot) {
        const float4* t8 = reinterpret_cast<const float4*>(args.tab_recv + 8 * 64 + 8 * q);
        const float4* t0 = reinterpret_cast<const float4*>(args.tab_recv + static_cast<int64_t>(p0 + min(grp, n - 1)) * 64 + 8 * q);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float4 v = t8[w];
          c8[2 * w] = v.x;
          s8[2 * w] = v.y;
          c8[2 * w + 1] = v.z;
          s8[2 * w + 1] = v.w;
          const float4 z = t0[w];
          cs[2 * w] = z.x;
          sn[2 * w] = z.y;
          cs[2 * w + 1] = z.z;
          sn[2 * w + 1] = z.w;
        }
      }
      int32_t rv = (lane < n) ? args.r2u[p0 + lane] : 0;
      for (int32_t base = 0; base < n; base += 64) {
        const int32_t rv_next = (base + 64 + lane < n) ? args.r2u[p0 + base + 64 + lane] : 0;
#pragma unroll 2
        for (int i = 0; i < 8; ++i) {
          const int32_t off = base + grp + 8 * i;
          const int ul = __shfl(rv, grp + 8 * i, 64) - u0;
          if (off < n) {
            const int swz = ((ul >> 2) & 1) << 5;
            const float* rowp = ep + ul * 128;
            const float4 x0 = *reinterpret_cast<const float4*>(rowp + ((8 * q) ^ swz));
            const float4 x1 = *reinterpret_cast<const float4*>(rowp + ((8 * q) ^ swz) + 4);
            const float4 y0 = *reinterpret_cast<const float4*>(rowp + ((64 + 8 * q) ^ swz));
            const float4 y1 = *reinterpret_cast<const float4*>(rowp + ((64 + 8 * q) ^ swz) + 4);
            float a[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            float b[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
            if (rot) {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float ra = a[e] * cs[e] - b[e] * sn[e];
                b[e] = a[e] * sn[e] + b[e] * cs[e];
                a[e] = ra;
              }
            }
            uint16_t* o = outp + static_cast<int64_t>(p0 + off) * args.f_out;
            *reinterpret_cast<u32x4*>(o) = u32x4{cvt_bf16x2(a[0], a[1]), cvt_bf16x2(a[2], a[3]),
                                                 cvt_bf16x2(a[4], a[5]), cvt_bf16x2(a[6], a[7])};
            *reinterpret_cast<u32x4*>(o + 64) = u32x4{cvt_bf16x2(b[0], b[1]), cvt_bf16x2(b[2], b[3]),
                                                      cvt_bf16x2(b[4], b[5]), cvt_bf16x2(b[6], b[7])};
          }
          if (rot) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float cn = cs[e] * c8[e] - sn[e] * s8[e];
              sn[e] = sn[e] * c8[e] + cs[e] * s8[e];
              cs[e] = cn;
            }
          }
        }
        rv = rv_next;
      }
    }
    // the next tile's first loads overwrite slots 0..2 (staging of waves 0..2)
    FT_COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    FT_COMPILER_FENCE();
  }
}

// ---------------------------------------------------------------- map preparation
// mode 0: bf16 -> fp16 (same layout); mode 1: fp32 -> [bf16 hi | bf16 lo];
// mode 2: fp32 -> [fp16 hi | fp16 lo].  Split maps double the K extent:
// out[l][o][f] = hi, out[l][o][F_in + f] = lo.
__global__ __launch_bounds__(256) void prepare_maps_kernel(const void* __restrict__ in, uint16_t* __restrict__ out,
                                                           int64_t rows, int32_t f_in, int32_t mode) {
  const int64_t total = rows * f_in;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (mode == 0) {
      out[i] = f32_to_f16_bits(bf16_to_f32(static_cast<const uint16_t*>(in)[i]));
    } else {
      const float x = static_cast<const float*>(in)[i];
      const int64_t r = i / f_in, f = i % f_in;
      uint16_t hi, lo;
      if (mode == 1) {
        hi = f32_to_bf16_rne(x);
        lo = f32_to_bf16_rne(x - bf16_to_f32(hi));
      } else {
        hi = f32_to_f16_bits(x);
        lo = f32_to_f16_bits(x - static_cast<float>(__builtin_bit_cast(_Float16, hi)));
      }
      out[r * 2 * f_in + f] = hi;
      out[r * 2 * f_in + f_in + f] = lo;
    }
  }
}

int launch_prepare_maps(const void* in, uint16_t* out, int64_t rows, int32_t f_in, int32_t mode, hipStream_t s) {
  const int64_t total = rows * f_in;
  if (total <= 0) return KVX_OK;
  int64_t blocks = ceil_div(total, 256);
  if (blocks > 32768) blocks = 32768;
  prepare_maps_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(in, out, rows, f_in, mode);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

int launch_flat(const FlatProblem& p, const FlatRole* roles, int n_roles, hipStream_t s) {
  if (p.recv_tokens <= 0 || n_roles <= 0) return KVX_OK;
  FlatKArgs a{};
  a.n_roles = n_roles;
  a.recv_layers = p.recv_layers;
  a.recv_tokens = p.recv_tokens;
  a.k_dim = p.k_dim;
  a.f_out = p.f_out;
  a.send_row = p.send_row;
  a.n_taps = p.n_taps;
  a.tab_recv = p.tab_recv;
  a.uniq = p.runs.uniq;
  a.run_begin = p.runs.run_begin;
  a.r2u = p.runs.recv_to_uniq;
  a.n_uniq = p.runs.n_uniq;
  if (p.k_dim % (4 * FT_BK) != 0 || p.send_row % FT_BK != 0) return KVX_ERR_UNSUPPORTED;
  for (int l = 0; l < p.recv_layers; ++l)
    for (int t = 0; t < p.n_taps; ++t)
      a.taps[l][t / 4] |= static_cast<uint32_t>(p.taps[l * p.n_taps + t] & 0xff) << (8 * (t % 4));
  int G = device_cu_count();
  G = G >= 8 ? (G / 8) * 8 : 8;
  // one launch per operand type (fp16 for rotated-back keys, bf16 otherwise)
  for (int f16 = 1; f16 >= 0; --f16) {
    FlatKArgs b = a;
    b.n_roles = 0;
    for (int j = 0; j < n_roles; ++j) {
      if (roles[j].a_f16 != f16) continue;
      const int k = b.n_roles++;
      b.a_src[k] = static_cast<const uint16_t*>(roles[j].a_src);
      b.a_layer_stride[k] = roles[j].a_layer_stride;
      b.a_compact[k] = roles[j].a_compact;
      b.a_f16[k] = roles[j].a_f16;
      b.wt[k] = static_cast<const uint16_t*>(roles[j].wt);
      b.bias[k] = roles[j].bias;
      b.out[k] = roles[j].out;
      b.rotate[k] = roles[j].rotate;
    }
    if (b.n_roles == 0) continue;
    if (f16)
      flat_gemm_kernel<true><<<G, FT_THREADS, 0, s>>>(b);
    else
      flat_gemm_kernel<false><<<G, FT_THREADS, 0, s>>>(b);
    KVX_LAUNCH_CHECK();
  }
  return KVX_OK;
}

}  // namespace kvx
