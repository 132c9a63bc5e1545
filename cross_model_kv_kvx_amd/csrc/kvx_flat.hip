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
//   * one workgroup of 8 waves per CU (two waves per SIMD, so one wave's
//     barrier wait or fragment-read latency is covered by the other's
//     matrix instructions); block tile 256 (rows) x 256 (outputs = two
//     128-wide heads), wave tile 64 x 128 (one head) built from 2 x 4 MFMA
//     32x32x16 accumulators;
//   * K advances 64 elements per step; the A part (256 rows x 64) and the W
//     part (256 outputs x 64) of a step are 32 KB each and go through a ring
//     of five 32 KB LDS parts (all 160 KB of LDS), filled by direct
//     global->LDS 16-byte loads: A rows are gathered per lane (sender token
//     of each run, or a compact rotated-back row) and W rows are read
//     output-major.  64 elements are one whole 128-byte line of each row, so
//     every L2 request is a full line (half-line requests halve the L2
//     throughput).  While step k is multiplied, W of step k+1 and A of steps
//     k+1 and k+2 are in flight.  Waves 0..3 (one per SIMD) issue all of a
//     step's loads and waves 4..7 none: the other wave of each SIMD never
//     waits behind a queued load issue, and waits on the vector-memory
//     counter only once per tile;
//   * inside each 128-byte LDS row the 16-byte chunks are XOR-swizzled by
//     (row / 2) mod 8 so fragment reads of consecutive rows hit distinct
//     banks;
//   * each part is a separate LDS array so the compiler can keep counted
//     vmcnt waits, and the only synchronisation per step is one s_barrier;
//   * the row tiles of all problems, in problem order, are grouped 8 at a
//     time (a group may hold the last row tiles of one problem and the first
//     of the next) x F_out/256 output tiles, and each group goes to
//     consecutive workgroups of one XCD (workgroups are dispatched round
//     robin over the 8 XCDs): the XCD's 32 concurrent tiles read 8 A slices
//     and 4 (or 8) W slices through its L2, and every A slice is read by one
//     group only;
//   * epilogue: each wave stages 32 rows x 128 outputs (bias added, fp32) in
//     its 16 KB share of parts 1..4, then walks the receiver rows of those
//     runs 8 at a time, rotating key pairs (c, c+64) at the receiver position
//     by a recurrence and storing 2 x 16 bytes of bf16 (nearest even) per
//     lane.  The receiver's own key normalisation ("Prefill-Free ...",
//     Methodology 2: keys are mapped before it and before RoPE) scales each
//     staged run row by its 1/RMS over the head and by the channel weights
//     before the rotation.

#include "kvx_internal.hpp"

namespace kvx {

constexpr int FT_M = 256;
constexpr int FT_N = 256;
constexpr int FT_BK = 64;
constexpr int FT_WAVES = 8;
constexpr int FT_THREADS = 64 * FT_WAVES;
constexpr int FT_GM = 8;                              // row tiles per L2 group
constexpr int FT_PART_ELEMS = FT_M * FT_BK;          // 16-bit elements of one ring part (32 KB)
static_assert(FT_M == FT_N, "A and W parts share one size");
constexpr int FT_ROWS_PER_LD = 8;                     // rows of one direct load (8 x 128 B)
constexpr int FT_LOADERS = 4;                         // waves 0..3 issue every direct load
constexpr int FT_A_LD = FT_M / FT_ROWS_PER_LD / FT_LOADERS;  // A loads per loading wave per step
constexpr int FT_B_LD = FT_N / FT_ROWS_PER_LD / FT_LOADERS;  // B loads per loading wave per step
constexpr int FT_EP_FLOATS = 32 * 128;                // staging of one wave (16 KB)
// fp8 maps: a W part holds 128 k of each of the 256 rows (32 KB, one whole
// 128-byte line per row) and serves two steps
constexpr int FT_W8_BK = 128;

struct FlatKArgs {
  const uint16_t* a_src[2];
  int64_t a_layer_stride[2];
  int32_t a_compact[2];
  int32_t a_f16[2];
  const void* wt[2];      // [L_R][F_out][K], K = k_dim: 16-bit operands, or fp8 E4M3 codes
  const float* wscale[2]; // fp8 maps: scale of each output [L_R][F_out]
  const float* bias[2];
  uint16_t* out[2];
  int32_t rotate[2];
  const float* knorm[2];  // key-normalisation weights [L_R][128] or null
  float knorm_eps;
  const int64_t* slot;     // output row of each receiver token, or null (row i)
  int64_t pool_rows;       // output rows per layer
  const int32_t* recv_pos; // rotary position of each receiver token, or null (i)
  int32_t pos_limit;
  int32_t n_roles;
  int32_t recv_layers, recv_tokens, k_dim, f_out, send_row, n_taps;
  const float2* tab_recv;
  const int32_t* uniq;
  const int32_t* run_begin;
  const int32_t* r2u;
  const int32_t* n_uniq;
  // receiver layer of the i-th problem of a role: layers whose taps share
  // sender layers follow one another, so their sender rows are read again
  // while still in the last-level cache
  uint8_t layer_order[MAX_LAYERS];
  // taps of layer l: bytes of taps[l][0] (taps 0..3) and taps[l][1] (4..6);
  // dword-packed so they are read with scalar loads
  uint32_t taps[MAX_LAYERS][2];
};

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Physical 16-byte chunk of logical chunk c in tile row r (128-byte rows of
// every part: 64 16-bit elements, or 128 fp8 codes of a W part).
__device__ __forceinline__ int ft_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

// Per-tile addressing of this thread's direct loads.  A load instruction
// covers 8 tile rows (1 KB of the stage); lane j lands at row +j/8, physical
// chunk j%8.  Loading wave w (< FT_LOADERS) loads row groups
// FT_A_LD*w .. +FT_A_LD of A and FT_B_LD*w .. +FT_B_LD of B.
struct TileAddr {
  const char* a_src;            // A source, layer 0
  int64_t a_ls;                 // bytes between A source layers (< 2^31)
  uint32_t taps0, taps1;        // sender layer of taps 0..3 and 4..6, one byte each
  const char* w_base;           // map rows n0 .. n0+255 of this layer
  uint32_t w_bytes;
  uint32_t a_off[FT_A_LD];      // byte offsets of the A rows (row * send_row + chunk)
  uint32_t b_off[FT_B_LD];      // byte offsets of the W rows
  int32_t spt;                  // K steps per tap (send_row / 64)
  int32_t n_taps;
  int32_t nk;                   // K steps of the problem
};

// Layer source of step k (fp32 maps split in two repeat the taps).
__device__ __forceinline__ uint32_t ft_layer(const TileAddr& ta, int k) {
  const int32_t tap = (k / ta.spt) % ta.n_taps;
  return ((tap < 4 ? ta.taps0 : ta.taps1) >> (8 * (tap & 3))) & 0xffu;
}

// A part of step k into `part` (steps past the end read an empty range).
__device__ __forceinline__ void ft_issue_a(const TileAddr& ta, int k, uint16_t* part) {
  const int wave = wave_id();
  const bool live = k < ta.nk;
  const __amdgpu_buffer_rsrc_t a_r = buf_rsrc(ta.a_src + static_cast<int64_t>(ft_layer(ta, k)) * ta.a_ls,
                                             live ? static_cast<uint32_t>(ta.a_ls) : 0u);
  const uint32_t a_soff = 2u * static_cast<uint32_t>((k % ta.spt) * FT_BK);
#pragma unroll
  for (int i = 0; i < FT_A_LD; ++i) dma16(a_r, ta.a_off[i], a_soff, part + (wave * FT_A_LD + i) * 512);
}

// W part of step k into `part` (16-bit maps).
__device__ __forceinline__ void ft_issue_b(const TileAddr& ta, int k, uint16_t* part) {
  const int wave = wave_id();
  const __amdgpu_buffer_rsrc_t w_r = buf_rsrc(ta.w_base, k < ta.nk ? ta.w_bytes : 0u);
  const uint32_t b_soff = 2u * static_cast<uint32_t>(k * FT_BK);
#pragma unroll
  for (int i = 0; i < FT_B_LD; ++i) dma16(w_r, ta.b_off[i], b_soff, part + (wave * FT_B_LD + i) * 512);
}

// The loads one K step issues (W of step k+1 into nb, A of step k+2 into
// na), spread over its sub-steps so the MFMAs of a wave do not wait behind
// a burst of load issues after each barrier.  W loads come first, then A
// loads: the next step's wait leaves exactly the A loads in flight.
struct StepLoads {
  __amdgpu_buffer_rsrc_t ar, br;
  uint32_t asoff, bsoff;
  uint16_t* na;
  uint16_t* nb;
};

// Position of the A part a step issues (step k + 2) inside the taps: the
// 64-element piece of the tap's row (a_in < spt) and the tap (a_tap <
// n_taps), carried from step to step instead of divided out each time.
struct ATap {
  int32_t a_in, a_tap;
};

__device__ __forceinline__ ATap ft_atap_start(const TileAddr& ta) {
  return ATap{2 % ta.spt, (2 / ta.spt) % ta.n_taps};
}

__device__ __forceinline__ void ft_atap_next(const TileAddr& ta, ATap& t) {
  if (++t.a_in == ta.spt) {
    t.a_in = 0;
    if (++t.a_tap == ta.n_taps) t.a_tap = 0;
  }
}

__device__ __forceinline__ StepLoads ft_step_loads(const TileAddr& ta, int k, const ATap& t, uint16_t* nb,
                                                   uint16_t* na) {
  StepLoads sl;
  const int kb = k + 1, ka = k + 2;
  sl.br = buf_rsrc(ta.w_base, kb < ta.nk ? ta.w_bytes : 0u);
  sl.bsoff = 2u * static_cast<uint32_t>(kb * FT_BK);
  const uint32_t layer = ((t.a_tap < 4 ? ta.taps0 : ta.taps1) >> (8 * (t.a_tap & 3))) & 0xffu;
  sl.ar = buf_rsrc(ta.a_src + static_cast<int64_t>(layer) * ta.a_ls, ka < ta.nk ? static_cast<uint32_t>(ta.a_ls) : 0u);
  sl.asoff = 2u * static_cast<uint32_t>(t.a_in * FT_BK);
  sl.na = na;
  sl.nb = nb;
  return sl;
}

// Load i of this wave's share of a step (W loads, then A loads).
__device__ __forceinline__ void ft_load(const TileAddr& ta, const StepLoads& sl, int i) {
  const int wave = wave_id();
  if (i < FT_B_LD)
    dma16(sl.br, ta.b_off[i], sl.bsoff, sl.nb + (wave * FT_B_LD + i) * 512);
  else
    dma16(sl.ar, ta.a_off[i - FT_B_LD], sl.asoff, sl.na + (wave * FT_A_LD + i - FT_B_LD) * 512);
}

// One K step from an A part and a W part: 4 x (2 A + 4 B fragment reads,
// 8 MFMAs).
template <bool F16, bool ISSUE = true>
__device__ __forceinline__ void ft_compute(const uint16_t* pa, const uint16_t* pb, f32x16 (&acc)[2][4],
                                           const TileAddr& ta, const StepLoads& sl) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;
  const char* sa = reinterpret_cast<const char*>(pa);
  const char* sb = reinterpret_cast<const char*>(pb);
  const int fr = lane & 31;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    // a loading wave issues four of its sixteen loads per sub-step (kept in
    // place: the scheduler would otherwise sink them to the end of the step)
    if constexpr (ISSUE) {
      constexpr int nps = (FT_A_LD + FT_B_LD) / 4;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < nps; ++j) ft_load(ta, sl, nps * kk + j);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int pc = ft_chunk(fr, 2 * kk + (lane >> 5)) << 4;
    u32x4 af[2], bfr[4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) af[mi] = *reinterpret_cast<const u32x4*>(sa + (wm * 64 + mi * 32 + fr) * 128 + pc);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      bfr[ni] = *reinterpret_cast<const u32x4*>(sb + (wn * 128 + ni * 32 + fr) * 128 + pc);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma32<F16>(af[mi], bfr[ni], acc[mi][ni]);
  }
}

// A loading wave waits until all but the last A part it issued have landed,
// then one barrier: the parts of the current step are complete and every
// wave has finished the previous step, whose two parts are now free.  The
// other waves issue no loads and only take the barrier.
template <bool LD>
__device__ __forceinline__ void ft_sync() {
  if constexpr (LD) KVX_WAIT_VM(FT_A_LD);
  KVX_COMPILER_FENCE();
  __builtin_amdgcn_s_barrier();
  KVX_COMPILER_FENCE();
}

// One step of the ring: A of step k is in part 2k mod 5, W in part
// 2k+1 mod 5; the step issues W of k+1 and A of k+2 into the two parts of
// step k-1.
// A whole step: loads spread over the sub-steps.
#define FT_STEP(K, PA, PB, NB, NA)                                    \
  {                                                                   \
    ft_sync<LD>();                                                    \
    const StepLoads sl = ft_step_loads(ta, (K), at, NB, NA);          \
    ft_atap_next(ta, at);                                             \
    ft_compute<F16, LD>(PA, PB, acc, ta, sl);                         \
  }
// A tail step: every load first, the products only while k < nk.
#define FT_TAIL(K, PA, PB, NB, NA)                                    \
  {                                                                   \
    ft_sync<LD>();                                                    \
    const StepLoads sl = ft_step_loads(ta, (K), at, NB, NA);          \
    ft_atap_next(ta, at);                                             \
    if constexpr (LD)                                                 \
      for (int i_ = 0; i_ < FT_B_LD + FT_A_LD; ++i_)                  \
        ft_load(ta, sl, i_);                                          \
    if ((K) < nk)                                                     \
      ft_compute<F16, false>(PA, PB, acc, ta, sl);                    \
  }

// K loop over nk >= 1 steps with A0, W0 and A1 already issued into parts 0,
// 1 and 2.  The part pattern repeats every five steps: whole groups of five
// run without branches, the remaining 1..4 steps (and the loads past the
// end, which read an empty buffer range so every wait keeps its count) run
// as a tail.  The loads still in flight at the end are drained before the
// parts are reused.  LD: this wave issues the loads.
template <bool F16, bool LD>
__device__ __forceinline__ void ft_kloop(const TileAddr& ta, int nk, uint16_t* p0, uint16_t* p1, uint16_t* p2,
                                         uint16_t* p3, uint16_t* p4, f32x16 (&acc)[2][4]) {
  int k = 0;
  ATap at = ft_atap_start(ta);
  for (; k + 5 <= nk; k += 5) {
    FT_STEP(k, p0, p1, p3, p4)
    FT_STEP(k + 1, p2, p3, p0, p1)
    FT_STEP(k + 2, p4, p0, p2, p3)
    FT_STEP(k + 3, p1, p2, p4, p0)
    FT_STEP(k + 4, p3, p4, p1, p2)
  }
  if (k < nk) {
    FT_TAIL(k, p0, p1, p3, p4)
    FT_TAIL(k + 1, p2, p3, p0, p1)
    FT_TAIL(k + 2, p4, p0, p2, p3)
    FT_TAIL(k + 3, p1, p2, p4, p0)
    FT_TAIL(k + 4, p3, p4, p1, p2)
  }
  if constexpr (LD) KVX_WAIT_VM(0);
}
#undef FT_TAIL
#undef FT_STEP

// ---------------------------------------------------------------- fp8 maps
// With fp8 maps the ring parts keep fixed roles: the A part of step k sits
// in part k mod 3 (p0..p2) and W part j, 128 k of each of the 256 rows
// (32 KB, one whole 128-byte line per row) serving steps 2j and 2j+1, in
// p3 or p4 (j mod 2).  W part j+1 is issued at step 2j, two steps before
// its first use; the A parts keep their two-step lead.  A loading wave
// issues 8 W and 8 A loads at an even step and 8 A loads at an odd one, so
// its wait leaves 8 loads in flight before an even step and 16 before an
// odd one.  The pattern repeats every 12 steps.

// W part j into `part`.
__device__ __forceinline__ void ft_issue_w8(const TileAddr& ta, int j, uint16_t* part) {
  const int wave = wave_id();
  const __amdgpu_buffer_rsrc_t w_r = buf_rsrc(ta.w_base, 2 * j < ta.nk ? ta.w_bytes : 0u);
  const uint32_t b_soff = static_cast<uint32_t>(j * FT_W8_BK);
#pragma unroll
  for (int i = 0; i < FT_B_LD; ++i) dma16(w_r, ta.b_off[i], b_soff, part + (wave * FT_B_LD + i) * 512);
}

// The loads of step k: W part k/2 + 1 into nb (even k) and A of step k + 2
// into na.
__device__ __forceinline__ StepLoads ft_step_loads8(const TileAddr& ta, int k, const ATap& t, uint16_t* nb,
                                                    uint16_t* na) {
  StepLoads sl;
  const int jb = (k >> 1) + 1, ka = k + 2;
  sl.br = buf_rsrc(ta.w_base, 2 * jb < ta.nk ? ta.w_bytes : 0u);
  sl.bsoff = static_cast<uint32_t>(jb * FT_W8_BK);
  const uint32_t layer = ((t.a_tap < 4 ? ta.taps0 : ta.taps1) >> (8 * (t.a_tap & 3))) & 0xffu;
  sl.ar = buf_rsrc(ta.a_src + static_cast<int64_t>(layer) * ta.a_ls, ka < ta.nk ? static_cast<uint32_t>(ta.a_ls) : 0u);
  sl.asoff = 2u * static_cast<uint32_t>(t.a_in * FT_BK);
  sl.na = na;
  sl.nb = nb;
  return sl;
}

// Load i of a loading wave's share of a step: at an even step the W loads
// and then the A loads, at an odd step the A loads only.
template <bool EVEN>
__device__ __forceinline__ void ft_load8(const TileAddr& ta, const StepLoads& sl, int i) {
  const int wave = wave_id();
  if (EVEN && i < FT_B_LD) {
    dma16(sl.br, ta.b_off[i], sl.bsoff, sl.nb + (wave * FT_B_LD + i) * 512);
  } else {
    const int ia = EVEN ? i - FT_B_LD : i;
    dma16(sl.ar, ta.a_off[ia], sl.asoff, sl.na + (wave * FT_A_LD + ia) * 512);
  }
}

// Eight fp8 E4M3 codes (two dwords, element e in byte e) as eight 16-bit
// operands of the A operand's type; exact (every E4M3 value is a normal bf16
// and a normal fp16).  The per-output scale is applied in the epilogue.
template <bool F16>
__device__ __forceinline__ u32x4 ft_fp8x8(uint32_t lo, uint32_t hi) {
  if constexpr (F16)
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true))};
  else
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
}

// One K step with fp8 maps, from an A part and half S of a W part.  The
// order of the 64 k inside a step is permuted (the same for both operands,
// so the contraction is unchanged): sub-step kk of lane half h takes logical
// 8-element chunk 4h + kk, so the W bytes a lane needs for sub-steps 2p and
// 2p+1 are one 16-byte chunk (4S + 2h + p of its 128-byte row) and one
// fragment read serves two sub-steps.  NPS loads are issued per sub-step.
template <bool F16, int NPS, int S>
__device__ __forceinline__ void ft_compute8(const uint16_t* pa, const uint16_t* pw, f32x16 (&acc)[2][4],
                                            const TileAddr& ta, const StepLoads& sl) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;
  const char* sa = reinterpret_cast<const char*>(pa);
  const char* sw = reinterpret_cast<const char*>(pw);
  const int fr = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {
    u32x4 braw[4];
    const int pcw = ft_chunk(fr, 4 * S + 2 * h + kp) << 4;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) braw[ni] = *reinterpret_cast<const u32x4*>(sw + (wn * 128 + ni * 32 + fr) * 128 + pcw);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kk = 2 * kp + sub;
      if constexpr (NPS > 0) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NPS; ++j) ft_load8<NPS == (FT_A_LD + FT_B_LD) / 4>(ta, sl, NPS * kk + j);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int pc = ft_chunk(fr, 4 * h + kk) << 4;
      u32x4 af[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = *reinterpret_cast<const u32x4*>(sa + (wm * 64 + mi * 32 + fr) * 128 + pc);
      // each W fragment is converted right before its two products, so one
      // converted fragment is live at a time
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const u32x4 bfr = sub == 0 ? ft_fp8x8<F16>(braw[ni][0], braw[ni][1]) : ft_fp8x8<F16>(braw[ni][2], braw[ni][3]);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) acc[mi][ni] = mfma32<F16>(af[mi], bfr, acc[mi][ni]);
      }
    }
  }
}

// Step k = (k - OFF) + OFF of the fp8 K loop, OFF = k mod 12 (fixes the
// parts and the wait count).  LIVE: k < nk is known; else the products run
// only while k < nk and the loads are issued before them.
template <bool F16, bool LD, int OFF, bool LIVE>
__device__ __forceinline__ void ft_step8(const TileAddr& ta, int k, int nk, ATap& at, uint16_t* const (&pa)[3],
                                         uint16_t* const (&pw)[2], f32x16 (&acc)[2][4]) {
  constexpr bool EVEN = (OFF & 1) == 0;
  constexpr int NLD = EVEN ? FT_A_LD + FT_B_LD : FT_A_LD;  // loads of a loading wave
  if constexpr (LD) KVX_WAIT_VM(EVEN ? FT_A_LD : FT_A_LD + FT_B_LD);
  KVX_COMPILER_FENCE();
  __builtin_amdgcn_s_barrier();
  KVX_COMPILER_FENCE();
  const StepLoads sl = ft_step_loads8(ta, k, at, pw[((OFF >> 1) + 1) & 1], pa[(OFF + 2) % 3]);
  ft_atap_next(ta, at);
  if constexpr (LIVE) {
    ft_compute8<F16, LD ? NLD / 4 : 0, OFF & 1>(pa[OFF % 3], pw[(OFF >> 1) & 1], acc, ta, sl);
  } else {
    if constexpr (LD)
      for (int i = 0; i < NLD; ++i) ft_load8<EVEN>(ta, sl, i);
    if (k < nk) ft_compute8<F16, 0, OFF & 1>(pa[OFF % 3], pw[(OFF >> 1) & 1], acc, ta, sl);
  }
}

// fp8 K loop over nk >= 1 steps with A0 in p0, W part 0 in p3 and A1 in p1
// already issued; whole groups of 12 steps run without branches, the rest
// as a 12-step tail (loads past the end read an empty range so every wait
// keeps its count), then the loads in flight are drained.
template <bool F16, bool LD>
__device__ __forceinline__ void ft_kloop8(const TileAddr& ta, int nk, uint16_t* p0, uint16_t* p1, uint16_t* p2,
                                          uint16_t* p3, uint16_t* p4, f32x16 (&acc)[2][4]) {
  uint16_t* const pa[3] = {p0, p1, p2};
  uint16_t* const pw[2] = {p3, p4};
  int k = 0;
  ATap at = ft_atap_start(ta);
  for (; k + 12 <= nk; k += 12) {
    ft_step8<F16, LD, 0, true>(ta, k, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 1, true>(ta, k + 1, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 2, true>(ta, k + 2, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 3, true>(ta, k + 3, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 4, true>(ta, k + 4, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 5, true>(ta, k + 5, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 6, true>(ta, k + 6, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 7, true>(ta, k + 7, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 8, true>(ta, k + 8, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 9, true>(ta, k + 9, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 10, true>(ta, k + 10, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 11, true>(ta, k + 11, nk, at, pa, pw, acc);
  }
  if (k < nk) {
    ft_step8<F16, LD, 0, false>(ta, k, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 1, false>(ta, k + 1, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 2, false>(ta, k + 2, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 3, false>(ta, k + 3, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 4, false>(ta, k + 4, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 5, false>(ta, k + 5, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 6, false>(ta, k + 6, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 7, false>(ta, k + 7, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 8, false>(ta, k + 8, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 9, false>(ta, k + 9, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 10, false>(ta, k + 10, nk, at, pa, pw, acc);
    ft_step8<F16, LD, 11, false>(ta, k + 11, nk, at, pa, pw, acc);
  }
  if constexpr (LD) KVX_WAIT_VM(0);
}

// Both operand types in one launch: the K loop is chosen per tile.  PLACED:
// output rows from the slot array and rotary positions per token (else row
// and position i).
template <bool PLACED, bool W8>
__global__ __attribute__((amdgpu_flat_work_group_size(FT_THREADS, FT_THREADS), amdgpu_waves_per_eu(2, 2))) void
flat_gemm_kernel(const FlatKArgs args) {
  __shared__ __attribute__((aligned(1024))) uint16_t p0[FT_PART_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t p1[FT_PART_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t p2[FT_PART_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t p3[FT_PART_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t p4[FT_PART_ELEMS];

  const int32_t U = *args.n_uniq;
  if (U <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;
  const int32_t mt = (U + FT_M - 1) / FT_M;
  const int32_t nt = args.f_out / FT_N;
  const int64_t per_p = static_cast<int64_t>(mt) * nt;
  const int64_t T = static_cast<int64_t>(args.n_roles) * args.recv_layers * per_p;
  const int32_t G = gridDim.x;
  const int32_t slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int32_t nk = args.k_dim / FT_BK;
  const int lrow = lane >> 3;  // row inside an 8-row load group
  // staging of this wave: half of part 1 + wave / 2
  uint16_t* const ep_part = wave < 2 ? p1 : (wave < 4 ? p2 : (wave < 6 ? p3 : p4));
  float* const ep = reinterpret_cast<float*>(ep_part) + (wave & 1) * FT_EP_FLOATS;

  const int64_t R = static_cast<int64_t>(args.n_roles) * args.recv_layers * mt;  // row tiles of all problems
  for (int64_t t = slot; t < T; t += G) {
    // group of FT_GM consecutive row tiles (of one problem or the end of one
    // and the start of the next) x all output tiles
    const int64_t g = t / (FT_GM * nt);
    const int32_t r2 = static_cast<int32_t>(t % (FT_GM * nt));
    const int32_t gm = static_cast<int32_t>(min(static_cast<int64_t>(FT_GM), R - g * FT_GM));
    const int32_t n0 = (r2 / gm) * FT_N;
    const int64_t mrow = g * FT_GM + r2 % gm;
    const int32_t p = static_cast<int32_t>(mrow / mt);
    const int32_t m0 = static_cast<int32_t>(mrow % mt) * FT_M;
    const int role = p / args.recv_layers;
    const int l = args.layer_order[p % args.recv_layers];

    TileAddr ta;
    ta.a_src = reinterpret_cast<const char*>(args.a_src[role]);
    ta.a_ls = 2 * args.a_layer_stride[role];
    ta.taps0 = args.taps[l][0];
    ta.taps1 = args.taps[l][1];
    ta.spt = args.send_row / FT_BK;
    ta.n_taps = args.n_taps;
    constexpr int wb = W8 ? 1 : 2;  // bytes per map element
    ta.w_base = static_cast<const char*>(args.wt[role]) + (static_cast<int64_t>(l) * args.f_out + n0) * args.k_dim * wb;
    ta.w_bytes = static_cast<uint32_t>(wb * FT_N * args.k_dim);
    ta.nk = nk;
    // the sender rows of this tile's A part: only the loading waves read
    // them, so the other waves issue no load at the tile start and nothing
    // makes them wait there for the previous tile's epilogue stores
    if (wave < FT_LOADERS) {
#pragma unroll
      for (int i = 0; i < FT_A_LD; ++i) {
        const int r = (wave * FT_A_LD + i) * FT_ROWS_PER_LD + lrow;
        int32_t u = m0 + r;
        u = u < U ? u : U - 1;
        const int32_t srow = args.a_compact[role] ? u : args.uniq[u];
        ta.a_off[i] = 2u * static_cast<uint32_t>(srow * args.send_row + ft_chunk(r, lane & 7) * 8);
      }
    } else {
#pragma unroll
      for (int i = 0; i < FT_A_LD; ++i) ta.a_off[i] = 0u;
    }
#pragma unroll
    for (int i = 0; i < FT_B_LD; ++i) {
      // W row r, 16-byte chunk: 8 elements of a 16-bit map, 16 of an fp8 map
      const int r = (wave * FT_B_LD + i) * FT_ROWS_PER_LD + lrow;
      ta.b_off[i] = static_cast<uint32_t>(r * args.k_dim * wb + ft_chunk(r, lane & 7) * 16);
    }

    // run starts of this wave's two epilogue phases, read now so they have
    // arrived when the K loop ends

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // prologue (loading waves): A0, W0 and A1 in flight.  The parts were
    // last used as staging before the final barrier of the previous tile, so
    // they are free.
    if constexpr (W8) {
      if (wave < FT_LOADERS) {
        ft_issue_a(ta, 0, p0);
        ft_issue_w8(ta, 0, p3);
        ft_issue_a(ta, 1, p1);
        if (args.a_f16[role])
          ft_kloop8<true, true>(ta, nk, p0, p1, p2, p3, p4, acc);
        else
          ft_kloop8<false, true>(ta, nk, p0, p1, p2, p3, p4, acc);
      } else {
        if (args.a_f16[role])
          ft_kloop8<true, false>(ta, nk, p0, p1, p2, p3, p4, acc);
        else
          ft_kloop8<false, false>(ta, nk, p0, p1, p2, p3, p4, acc);
      }
    } else {
      if (wave < FT_LOADERS) {
        ft_issue_a(ta, 0, p0);
        ft_issue_b(ta, 0, p1);
        ft_issue_a(ta, 1, p2);
        if (args.a_f16[role])
          ft_kloop<true, true>(ta, nk, p0, p1, p2, p3, p4, acc);
        else
          ft_kloop<false, true>(ta, nk, p0, p1, p2, p3, p4, acc);
      } else {
        if (args.a_f16[role])
          ft_kloop<true, false>(ta, nk, p0, p1, p2, p3, p4, acc);
        else
          ft_kloop<false, false>(ta, nk, p0, p1, p2, p3, p4, acc);
      }
    }

    // ------------------------------------------------------------ epilogue
    // Each wave owns 64 unique rows x one 128-wide head, written in two
    // phases of 32 unique rows (one accumulator row block) staged with bias
    // in fp32.  The phase's receiver rows P0 .. P1-1 are walked by 8 lane
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
    float wsc[4];   // fp8 maps: scale of those columns
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t oc = static_cast<int64_t>(l) * args.f_out + n0 + wn * 128 + ni * 32 + (lane & 31);
      bcol[ni] = bias ? bias[oc] : 0.0f;
      wsc[ni] = W8 ? args.wscale[role][oc] : 1.0f;
    }
    const bool rot = args.rotate[role] != 0;
    // the receiver's key normalisation: weights of this lane's pair members
    // (channels 8q.. and 64 + 8q.., read where used: L1-resident)
    const float* kn = args.knorm[role];
    const float4* g4 = kn ? reinterpret_cast<const float4*>(kn + static_cast<int64_t>(l) * 128 + 8 * q) : nullptr;
    uint16_t* outp = args.out[role] + static_cast<int64_t>(l) * args.pool_rows * args.f_out + n0 + col;
    const int32_t* rpos = (PLACED && rot) ? args.recv_pos : nullptr;  // per-token positions, no recurrence
    // every wave has finished reading the parts
    KVX_COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    KVX_COMPILER_FENCE();
    // run index of the first 64 receiver rows of each phase, requested
    // before the staging so the stores need not wait for them
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      const int32_t u0 = m0 + wm * 64 + 32 * ph;
      // stage the phase's 32 rows (columns XOR 32 on rows with bit 2 set so
      // the two half-waves hit different banks); the scheduling barrier keeps
      // the accumulator reads of a phase here
      __builtin_amdgcn_sched_barrier(0);
      KVX_COMPILER_FENCE();
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int cc = (ni * 32 + (lane & 31)) ^ (((row >> 2) & 1) << 5);
          if constexpr (W8)
            ep[row * 128 + cc] = acc[ph][ni][r] * wsc[ni] + bcol[ni];
          else
            ep[row * 128 + cc] = acc[ph][ni][r] + bcol[ni];
        }
      KVX_COMPILER_FENCE();  // LDS operations of one wave execute in order
      __builtin_amdgcn_sched_barrier(0);
      if (u0 >= U) continue;
      // 1 / RMS of each staged row (lanes 2r and 2r+1 sum the two halves of
      // row r; the column swizzle only permutes a row)
      float inv = 1.0f;
      if (kn) {
        const float4* h4 = reinterpret_cast<const float4*>(ep + (lane >> 1) * 128 + 64 * (lane & 1));
        float ss = 0.0f;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
          const float4 v = h4[w];
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
        ss += __shfl_xor(ss, 1, 64);
        inv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + args.knorm_eps);
      }
      const int32_t p0 = args.run_begin[u0];
      const int32_t n = args.run_begin[min(u0 + 32, U)] - p0;
      float cs[8], sn[8], c8[8], s8[8];
      if (rot && !rpos) {
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
          const float sc = __shfl(inv, 2 * min(max(ul, 0), 31), 64);  // unconditional: all lanes take part
          if (off < n) {
            const int swz = ((ul >> 2) & 1) << 5;
            const float* rowp = ep + ul * 128;
            const float4 x0 = *reinterpret_cast<const float4*>(rowp + ((8 * q) ^ swz));
            const float4 x1 = *reinterpret_cast<const float4*>(rowp + ((8 * q) ^ swz) + 4);
            const float4 y0 = *reinterpret_cast<const float4*>(rowp + ((64 + 8 * q) ^ swz));
            const float4 y1 = *reinterpret_cast<const float4*>(rowp + ((64 + 8 * q) ^ swz) + 4);
            float a[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            float b[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
            if (kn) {
              const float4 u0 = g4[0], u1 = g4[1], v0 = g4[16], v1 = g4[17];
              const float ga[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
              const float gb[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                a[e] *= sc * ga[e];
                b[e] *= sc * gb[e];
              }
            }
            if (rpos) {
              // position of this receiver token (several sequences): table row
              int32_t pp = rpos[p0 + off];
              pp = pp < 0 ? 0 : (pp >= args.pos_limit ? args.pos_limit - 1 : pp);
              const float4* tp = reinterpret_cast<const float4*>(args.tab_recv + static_cast<int64_t>(pp) * 64 + 8 * q);
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const float4 t = tp[w];  // (cos, sin) of pairs 2w and 2w+1
                const float ra0 = a[2 * w] * t.x - b[2 * w] * t.y;
                b[2 * w] = a[2 * w] * t.y + b[2 * w] * t.x;
                a[2 * w] = ra0;
                const float ra1 = a[2 * w + 1] * t.z - b[2 * w + 1] * t.w;
                b[2 * w + 1] = a[2 * w + 1] * t.w + b[2 * w + 1] * t.z;
                a[2 * w + 1] = ra1;
              }
            } else if (rot) {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float ra = a[e] * cs[e] - b[e] * sn[e];
                b[e] = a[e] * sn[e] + b[e] * cs[e];
                a[e] = ra;
              }
            }
            int64_t orow = p0 + off;
            if (PLACED && args.slot) orow = args.slot[p0 + off];
            if (orow >= 0 && orow < args.pool_rows) {
              uint16_t* o = outp + orow * args.f_out;
              // streaming stores: the translated rows are not read again here,
              // so they should not evict the maps and sender rows that the
              // other tiles still read through L2 and the last-level cache
              __builtin_nontemporal_store(u32x4{cvt_bf16x2(a[0], a[1]), cvt_bf16x2(a[2], a[3]),
                                                cvt_bf16x2(a[4], a[5]), cvt_bf16x2(a[6], a[7])},
                                          reinterpret_cast<u32x4*>(o));
              __builtin_nontemporal_store(u32x4{cvt_bf16x2(b[0], b[1]), cvt_bf16x2(b[2], b[3]),
                                                cvt_bf16x2(b[4], b[5]), cvt_bf16x2(b[6], b[7])},
                                          reinterpret_cast<u32x4*>(o + 64));
            }
          }
          if (rot && !rpos) {
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
    // the next tile's first loads overwrite parts 1 and 2 (staging)
    KVX_COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    KVX_COMPILER_FENCE();
  }
}

// ---------------------------------------------------------------- map preparation
// The caller's maps are row-major [batch][R][C] (R inputs, C outputs,
// y = x W); the kernels read them output-major, [batch][C][m R], in the
// operand type of the role (see MapMode).  The split modes write the high
// half at [o][f] and the low half at [o][R + f]: W = hi + lo to about 2^-16
// relative (bf16) or better (fp16), and the K loop runs over 2 R.  Every
// conversion rounds to nearest even.  64 x 64 tiles through LDS: the reads
// run along C and the writes along R.
__global__ __launch_bounds__(256) void transpose_maps_kernel(const void* __restrict__ in, void* __restrict__ out,
                                                             int32_t R, int32_t C, int32_t mode) {
  __shared__ float tile[64][65];
  const int64_t b = blockIdx.z;
  const int32_t r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tc = threadIdx.x & 63, tr = threadIdx.x >> 6;
  const bool in_f32 = mode == TM_F32 || mode == TM_SPLIT_BF16 || mode == TM_SPLIT_F16;
#pragma unroll 4
  for (int r = tr; r < 64; r += 4) {
    const int32_t rr = r0 + r, cc = c0 + tc;
    float v = 0.0f;
    if (rr < R && cc < C) {
      const int64_t i = (b * R + rr) * C + cc;
      v = in_f32 ? static_cast<const float*>(in)[i] : bf16_to_f32(static_cast<const uint16_t*>(in)[i]);
    }
    tile[r][tc] = v;
  }
  __syncthreads();
  const bool split = mode == TM_SPLIT_BF16 || mode == TM_SPLIT_F16;
  const int64_t row = split ? 2 * static_cast<int64_t>(R) : R;
#pragma unroll 4
  for (int c = tr; c < 64; c += 4) {
    const int32_t cc = c0 + c, rr = r0 + tc;
    if (rr >= R || cc >= C) continue;
    const float v = tile[tc][c];
    const int64_t o = (b * C + cc) * row + rr;
    if (mode == TM_F32) {
      static_cast<float*>(out)[o] = v;
    } else if (mode == TM_BF16) {
      static_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(v);  // exact: v came from bf16
    } else if (mode == TM_F16) {
      static_cast<uint16_t*>(out)[o] = f32_to_f16_bits(v);
    } else if (mode == TM_SPLIT_BF16) {
      const uint16_t hi = f32_to_bf16_rne(v);
      static_cast<uint16_t*>(out)[o] = hi;
      static_cast<uint16_t*>(out)[o + R] = f32_to_bf16_rne(v - bf16_to_f32(hi));
    } else {
      const uint16_t hi = f32_to_f16_bits(v);
      static_cast<uint16_t*>(out)[o] = hi;
      static_cast<uint16_t*>(out)[o + R] =
          f32_to_f16_bits(v - static_cast<float>(__builtin_bit_cast(_Float16, hi)));
    }
  }
}

int launch_transpose_maps(const void* in, void* out, int64_t batch, int32_t R, int32_t C, int32_t mode,
                          hipStream_t s) {
  if (batch <= 0 || R <= 0 || C <= 0) return KVX_OK;
  if (batch > 65535) return KVX_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(ceil_div(C, 64)), static_cast<unsigned>(ceil_div(R, 64)),
                  static_cast<unsigned>(batch));
  transpose_maps_kernel<<<grid, 256, 0, s>>>(in, out, R, C, mode);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// ---------------------------------------------------------------- fp8 map storage
// "Cross-Model KV Cache Transfer in Production" (Implementation Guidelines,
// precision): weights may be stored quantised (FP8) while the product keeps
// 16-bit operands.  OCP E4M3 (bias 7, 3 mantissa bits, no infinities, 448
// the largest finite value): with E = max(exponent(|v|), -6), neighbouring
// codes at |v| are 2^(E-3) apart, n = rint(|v| 2^(3-E)) in 0..16 (exact
// power-of-two scaling, then nearest even) and the code is
// 8 (E + 7) + n - 8, which also covers the subnormals (E = -6, n < 8) and a
// round-up into the next binade (n = 16).  Codes past 448 saturate there;
// non-finite inputs saturate too.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a <= 512.0f)) return sign | 0x7eu;
  int e = static_cast<int>((u >> 23) & 0xffu) - 127;
  if (e < -6) e = -6;
  const int n = static_cast<int>(rintf(ldexpf(a, 3 - e)));
  int code = 8 * (e + 7) + n - 8;
  if (code > 0x7e) code = 0x7e;
  return sign | static_cast<uint32_t>(code);
}

// One workgroup per 16 consecutive outputs o of one map w[f][o] (row-major
// [f_in][f_out]): amax over f (order-free), scale = amax / 448 (1 when that
// is zero), codes of w / scale; both divisions correctly rounded.  Codes go
// out output-major, q[o][f], staged 1024 inputs at a time in LDS so the
// writes run along f.
constexpr int QZ_OUT = 16;
constexpr int QZ_CHUNK = 1024;
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const float* __restrict__ w, int32_t f_in, int32_t f_out,
                                                           uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[16][QZ_OUT + 1];
  __shared__ float sc_s[QZ_OUT];
  __shared__ uint8_t codes[QZ_OUT][QZ_CHUNK + 16];
  const int64_t b = blockIdx.y;
  const int32_t o0 = blockIdx.x * QZ_OUT;
  const int oc = threadIdx.x % QZ_OUT, rg = threadIdx.x / QZ_OUT;  // output, row group
  const int32_t o = o0 + oc;
  const float* wb = w + b * f_in * static_cast<int64_t>(f_out);
  float m = 0.0f;
  if (o < f_out)
    for (int32_t f = rg; f < f_in; f += 16) m = fmaxf(m, fabsf(wb[static_cast<int64_t>(f) * f_out + o]));
  red[rg][oc] = m;
  __syncthreads();
  if (threadIdx.x < QZ_OUT) {
    float mm = 0.0f;
    for (int g = 0; g < 16; ++g) mm = fmaxf(mm, red[g][threadIdx.x]);
    float sc = __fdiv_rn(mm, 448.0f);
    if (!(sc > 0.0f)) sc = 1.0f;
    sc_s[threadIdx.x] = sc;
    if (o0 + static_cast<int32_t>(threadIdx.x) < f_out) scale[b * f_out + o0 + threadIdx.x] = sc;
  }
  __syncthreads();
  const float sc = sc_s[oc];
  for (int32_t f0 = 0; f0 < f_in; f0 += QZ_CHUNK) {
    const int32_t n = min(QZ_CHUNK, f_in - f0);
    for (int32_t fl = rg; fl < n; fl += 16)
      codes[oc][fl] = o < f_out ? static_cast<uint8_t>(e4m3_rne(__fdiv_rn(wb[static_cast<int64_t>(f0 + fl) * f_out + o], sc)))
                                : 0;
    __syncthreads();
    for (int32_t i = threadIdx.x; i < QZ_OUT * n; i += 256) {
      const int32_t r = i / n, fl = i % n;
      if (o0 + r < f_out) q[(b * f_out + o0 + r) * static_cast<int64_t>(f_in) + f0 + fl] = codes[r][fl];
    }
    __syncthreads();
  }
}

int launch_quantize_fp8(const float* w, int64_t count, int32_t f_in, int32_t f_out, uint8_t* q, float* scale,
                        hipStream_t s) {
  if (count <= 0) return KVX_OK;
  if (count > 65535) return KVX_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(ceil_div(f_out, QZ_OUT)), static_cast<unsigned>(count));
  quantize_fp8_kernel<<<grid, 256, 0, s>>>(w, f_in, f_out, q, scale);
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
  if (p.k_dim % FT_BK != 0 || p.k_dim < FT_BK || p.send_row % FT_BK != 0 || p.f_out % FT_N != 0)
    return KVX_ERR_UNSUPPORTED;
  for (int l = 0; l < p.recv_layers; ++l)
    for (int t = 0; t < p.n_taps; ++t)
      a.taps[l][t / 4] |= static_cast<uint32_t>(p.taps[l * p.n_taps + t] & 0xff) << (8 * (t % 4));
  // problem order inside a role: from layer 0, each next layer is the
  // unvisited one sharing the most sender layers with the current one (the
  // nearest on ties)
  {
    bool used[MAX_LAYERS] = {false};
    int cur = 0;
    used[0] = true;
    a.layer_order[0] = 0;
    for (int i = 1; i < p.recv_layers; ++i) {
      int best = -1, best_shared = -1, best_dist = 0;
      for (int c = 0; c < p.recv_layers; ++c) {
        if (used[c]) continue;
        int shared = 0;
        for (int t = 0; t < p.n_taps; ++t) {
          const int32_t sl = p.taps[c * p.n_taps + t];
          bool seen = false;  // count each sender layer of c once
          for (int u = 0; u < t; ++u) seen = seen || p.taps[c * p.n_taps + u] == sl;
          if (seen) continue;
          for (int u = 0; u < p.n_taps; ++u)
            if (p.taps[cur * p.n_taps + u] == sl) {
              ++shared;
              break;
            }
        }
        const int dist = c > cur ? c - cur : cur - c;
        if (shared > best_shared || (shared == best_shared && dist < best_dist)) {
          best = c;
          best_shared = shared;
          best_dist = dist;
        }
      }
      used[best] = true;
      a.layer_order[i] = static_cast<uint8_t>(best);
      cur = best;
    }
  }
  int G = device_cu_count();
  G = G >= 8 ? (G / 8) * 8 : 8;
  for (int j = 0; j < n_roles; ++j) {
    a.a_src[j] = static_cast<const uint16_t*>(roles[j].a_src);
    a.a_layer_stride[j] = roles[j].a_layer_stride;
    a.a_compact[j] = roles[j].a_compact;
    a.a_f16[j] = roles[j].a_f16;
    a.wt[j] = roles[j].wt;
    a.wscale[j] = roles[j].wscale;
    a.bias[j] = roles[j].bias;
    a.out[j] = roles[j].out;
    a.rotate[j] = roles[j].rotate;
    a.knorm[j] = roles[j].knorm;
  }
  a.knorm_eps = p.knorm_eps;
  a.slot = p.slot;
  a.pool_rows = p.pool_rows;
  a.recv_pos = p.recv_pos;
  a.pos_limit = p.pos_limit;
  const bool placed = p.slot || p.recv_pos || p.pool_rows != p.recv_tokens;
  if (p.w8) {
    for (int j = 0; j < n_roles; ++j)
      if (!roles[j].wscale) return KVX_ERR_INVALID;
    if (placed)
      flat_gemm_kernel<true, true><<<G, FT_THREADS, 0, s>>>(a);
    else
      flat_gemm_kernel<false, true><<<G, FT_THREADS, 0, s>>>(a);
  } else if (placed) {
    flat_gemm_kernel<true, false><<<G, FT_THREADS, 0, s>>>(a);
  } else {
    flat_gemm_kernel<false, false><<<G, FT_THREADS, 0, s>>>(a);
  }
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

}  // namespace kvx
