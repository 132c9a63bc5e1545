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
// problems, each T[U x F_out] = A[U x F_in] * W^T + b:
//   * block tile 256 (rows) x 256 (outputs, two 128-wide heads), 4 waves of
//     128 x 128 built from 32x32x16 MFMAs with fp32 accumulation;
//   * K loop over F_in in steps of 64 (32 when the map is fp32 and is split
//     into a high and a low half), A rows gathered from the sender cache (or
//     from rotated-back fp16 key rows), W rows read output-major; both staged
//     through double-buffered, padded LDS (row stride + 16 bytes, no bank
//     conflicts for the 16-byte fragment reads);
//   * tiles of one problem are grouped 8 (rows) x F_out/256 (outputs) and one
//     group goes to the 32 blocks of one XCD (blocks are dispatched round
//     robin over the 8 XCDs), so A and W slices are shared in that XCD's L2;
//   * epilogue: each wave stages 32 rows x 128 outputs in LDS, then 8 lanes
//     per receiver row add the bias, rotate pairs (c, c+64) at the receiver
//     position and store 2 x 16 bytes of bf16 (nearest even).

#include "kvx_internal.hpp"

namespace kvx {

constexpr int FT_M = 256;
constexpr int FT_N = 256;
constexpr int FT_THREADS = 256;

struct FlatKArgs {
  const void* a_src[2];
  int64_t a_layer_stride[2];
  int32_t a_compact[2];
  const void* wt[2];
  const float* bias[2];
  uint16_t* out[2];
  int32_t rotate[2];
  int32_t a_f16[2];
  int32_t n_roles;
  int32_t recv_layers, recv_tokens, f_in, f_out, send_row, n_taps;
  const float2* tab_recv;
  const int32_t* uniq;
  const int32_t* run_begin;
  const int32_t* r2u;
  const int32_t* n_uniq;
  uint8_t taps[MAX_LAYERS * MAX_TAPS];
};

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// bf16 bits -> fp16 bits (exact for the magnitudes a map holds; rounds to
// nearest even below the fp16 normal range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16(bf16lo(w), bf16hi(w));
}

template <int SPLIT, bool F16, bool WF32>
__device__ __forceinline__ void flat_tile(const FlatKArgs& args, uint16_t* smem, int role, int l, int32_t m0,
                                          int32_t n0, int32_t U);

template <int SPLIT, bool WF32>
__global__ __launch_bounds__(FT_THREADS, 1) void flat_gemm_kernel(const FlatKArgs args) {
  constexpr int BK = 64 / SPLIT;
  constexpr int LDR = BK + 8;
  constexpr int STAGE = FT_M * LDR + SPLIT * FT_N * LDR;
  static_assert(2 * STAGE * 2 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int32_t U = *args.n_uniq;
  if (U <= 0) return;
  const int32_t mt = (U + FT_M - 1) / FT_M;
  const int32_t nt = args.f_out / FT_N;
  const int64_t per_p = static_cast<int64_t>(mt) * nt;
  const int64_t T = static_cast<int64_t>(args.n_roles) * args.recv_layers * per_p;
  const int32_t G = gridDim.x;
  const int32_t slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  for (int64_t t = slot; t < T; t += G) {
    const int32_t p = static_cast<int32_t>(t / per_p);
    const int32_t rr = static_cast<int32_t>(t % per_p);
    const int32_t mg = rr / (8 * nt);
    const int32_t r2 = rr % (8 * nt);
    const int32_t gm = min(8, mt - mg * 8);
    const int32_t n_idx = r2 / gm;
    const int32_t m_idx = mg * 8 + r2 % gm;
    const int role = p / args.recv_layers;
    const int l = p % args.recv_layers;
    if (args.a_f16[role])
      flat_tile<SPLIT, true, WF32>(args, smem, role, l, m_idx * FT_M, n_idx * FT_N, U);
    else
      flat_tile<SPLIT, false, WF32>(args, smem, role, l, m_idx * FT_M, n_idx * FT_N, U);
  }
}

// One 256 x 256 output tile: K loop, then the run-expanding epilogue.
template <int SPLIT, bool F16, bool WF32>
__device__ __forceinline__ void flat_tile(const FlatKArgs& args, uint16_t* smem, int role, int l, int32_t m0,
                                          int32_t n0, int32_t U) {
  constexpr int BK = 64 / SPLIT;        // K elements per stage
  constexpr int LDR = BK + 8;           // LDS row stride in 16-bit elements
  constexpr int A_ELEMS = FT_M * LDR;
  constexpr int B_ELEMS = FT_N * LDR;
  constexpr int STAGE = A_ELEMS + SPLIT * B_ELEMS;
  constexpr int CPR = BK / 8;           // 16-byte chunks per A row per stage
  constexpr int A_PASSES = CPR;         // rows per pass = 256 / CPR
  constexpr int A_RSTEP = FT_M / CPR;
  // W chunks: bf16 -> 8 elements per 16 bytes; fp32 -> 4 elements.
  constexpr int WCE = WF32 ? 4 : 8;
  constexpr int CPRB = BK / WCE;
  constexpr int B_PASSES = CPRB;
  constexpr int B_RSTEP = FT_N / CPRB;
  static_assert(!WF32 || SPLIT == 2, "fp32 maps are split in two");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int32_t nk = args.f_in / BK;
  const int a_c = tid % CPR;
  const int a_r = tid / CPR;
  const int b_c = tid % CPRB;
  const int b_r = tid / CPRB;
  {
    const uint16_t* a_src = static_cast<const uint16_t*>(args.a_src[role]);
    const int64_t a_ls = args.a_layer_stride[role];
    const int a_compact = args.a_compact[role];
    int64_t a_row_off[A_PASSES];
#pragma unroll
    for (int i = 0; i < A_PASSES; ++i) {
      int32_t u = m0 + a_r + i * A_RSTEP;
      u = u < U ? u : U - 1;
      const int32_t srow = a_compact ? u : args.uniq[u];
      a_row_off[i] = static_cast<int64_t>(srow) * args.send_row + a_c * 8;
    }
    const uint8_t* tp = args.taps + l * MAX_TAPS;
    const int64_t w_base = (static_cast<int64_t>(l) * args.f_out + n0) * args.f_in;

    u32x4 ra[A_PASSES];
    u32x4 rb[B_PASSES];

    auto load_global = [&](int ks) {
      const int32_t f0 = ks * BK;
      const int32_t tap = f0 / args.send_row;
      const int32_t w = f0 - tap * args.send_row;
      const uint16_t* ab = a_src + static_cast<int64_t>(tp[tap]) * a_ls + w;
#pragma unroll
      for (int i = 0; i < A_PASSES; ++i)
        ra[i] = *reinterpret_cast<const u32x4*>(ab + a_row_off[i]);
      if constexpr (WF32) {
        const float* wb = static_cast<const float*>(args.wt[role]) + w_base + f0 + b_c * WCE;
#pragma unroll
        for (int i = 0; i < B_PASSES; ++i)
          rb[i] = *reinterpret_cast<const u32x4*>(wb + static_cast<int64_t>(b_r + i * B_RSTEP) * args.f_in);
      } else {
        const uint16_t* wb = static_cast<const uint16_t*>(args.wt[role]) + w_base + f0 + b_c * WCE;
#pragma unroll
        for (int i = 0; i < B_PASSES; ++i)
          rb[i] = *reinterpret_cast<const u32x4*>(wb + static_cast<int64_t>(b_r + i * B_RSTEP) * args.f_in);
      }
    };

    auto store_lds = [&](int stage) {
      uint16_t* As = smem + stage * STAGE;
      uint16_t* Bs = As + A_ELEMS;
#pragma unroll
      for (int i = 0; i < A_PASSES; ++i)
        *reinterpret_cast<u32x4*>(As + (a_r + i * A_RSTEP) * LDR + a_c * 8) = ra[i];
#pragma unroll
      for (int i = 0; i < B_PASSES; ++i) {
        const int row = b_r + i * B_RSTEP;
        if constexpr (WF32) {
          const float* f = reinterpret_cast<const float*>(&rb[i]);
          uint32_t hi[2], lo[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float x0 = f[2 * e], x1 = f[2 * e + 1];
            if constexpr (F16) {
              const uint32_t h = pack_f16(x0, x1);
              const float h0 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
              const float h1 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h >> 16)));
              hi[e] = h;
              lo[e] = pack_f16(x0 - h0, x1 - h1);
            } else {
              const uint32_t h = pack_bf16(x0, x1);
              hi[e] = h;
              lo[e] = pack_bf16(x0 - bf16lo(h), x1 - bf16hi(h));
            }
          }
          *reinterpret_cast<u32x2*>(Bs + row * LDR + b_c * WCE) = u32x2{hi[0], hi[1]};
          *reinterpret_cast<u32x2*>(Bs + B_ELEMS + row * LDR + b_c * WCE) = u32x2{lo[0], lo[1]};
        } else {
          u32x4 v = rb[i];
          if constexpr (F16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = bf16x2_to_f16x2(v[e]);
          }
          *reinterpret_cast<u32x4*>(Bs + row * LDR + b_c * WCE) = v;
        }
      }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    load_global(0);
    store_lds(0);
    __syncthreads();

    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;
    for (int ks = 0; ks < nk; ++ks) {
      const int stage = ks & 1;
      if (ks + 1 < nk) load_global(ks + 1);
      const uint16_t* As = smem + stage * STAGE;
      const uint16_t* Bs = As + A_ELEMS;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        u32x4 af[4], bfr[SPLIT][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          af[mi] = *reinterpret_cast<const u32x4*>(As + (wm * 128 + mi * 32 + frag_row) * LDR + kk * 16 + frag_k);
#pragma unroll
        for (int sp = 0; sp < SPLIT; ++sp)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            bfr[sp][ni] = *reinterpret_cast<const u32x4*>(Bs + sp * B_ELEMS + (wn * 128 + ni * 32 + frag_row) * LDR + kk * 16 + frag_k);
#pragma unroll
        for (int sp = 0; sp < SPLIT; ++sp)
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma32<F16>(af[mi], bfr[sp][ni], acc[mi][ni]);
      }
      if (ks + 1 < nk) store_lds(stage ^ 1);
      __syncthreads();
    }

    // ------------------------------------------------------------ epilogue
    constexpr int EPI_LD = 132;  // floats per staged row (128 + 4 pad)
    float* ep = reinterpret_cast<float*>(smem) + wave * 32 * EPI_LD;
    const int q = lane & 7;
    const int col = wn * 128 + 8 * q;  // tile column of the first pair member
    const float* bias = args.bias[role];
    float bA[8], bB[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bA[e] = bias ? bias[static_cast<int64_t>(l) * args.f_out + n0 + col + e] : 0.0f;
      bB[e] = bias ? bias[static_cast<int64_t>(l) * args.f_out + n0 + col + 64 + e] : 0.0f;
    }
    const int rot = args.rotate[role];
    uint16_t* outp = args.out[role] + static_cast<int64_t>(l) * args.recv_tokens * args.f_out + n0 + col;

#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          ep[row * EPI_LD + ni * 32 + (lane & 31)] = acc[mi][ni][r];
        }
      __syncthreads();
      const int32_t u0 = m0 + wm * 128 + mi * 32;
      if (u0 < U) {
        const int32_t rb0 = args.run_begin[u0];
        const int32_t rb1 = args.run_begin[min(u0 + 32, U)];
        for (int32_t rho = rb0 + (lane >> 3); rho < rb1; rho += 8) {
          const int ul = args.r2u[rho] - u0;
          const float4* src = reinterpret_cast<const float4*>(ep + ul * EPI_LD + 8 * q);
          const float4 x0 = src[0], x1 = src[1];
          const float4 y0 = src[16], y1 = src[17];  // +64 floats
          float a[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          float b[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            a[e] += bA[e];
            b[e] += bB[e];
          }
          if (rot) {
            const float4* tb = reinterpret_cast<const float4*>(args.tab_recv + static_cast<int64_t>(rho) * 64 + 8 * q);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const float4 cs = tb[w];
              const float a0 = a[2 * w] * cs.x - b[2 * w] * cs.y;
              const float b0 = a[2 * w] * cs.y + b[2 * w] * cs.x;
              const float a1 = a[2 * w + 1] * cs.z - b[2 * w + 1] * cs.w;
              const float b1 = a[2 * w + 1] * cs.w + b[2 * w + 1] * cs.z;
              a[2 * w] = a0;
              b[2 * w] = b0;
              a[2 * w + 1] = a1;
              b[2 * w + 1] = b1;
            }
          }
          uint16_t* o = outp + static_cast<int64_t>(rho) * args.f_out;
          *reinterpret_cast<u32x4*>(o) =
              u32x4{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(a[4], a[5]), pack_bf16(a[6], a[7])};
          *reinterpret_cast<u32x4*>(o + 64) =
              u32x4{pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3]), pack_bf16(b[4], b[5]), pack_bf16(b[6], b[7])};
        }
      }
      __syncthreads();
    }
  }
}

template <int SPLIT, bool WF32>
static int launch_flat_t(const FlatKArgs& a, hipStream_t s) {
  int G = device_cu_count();
  G = G >= 8 ? (G / 8) * 8 : 8;
  flat_gemm_kernel<SPLIT, WF32><<<G, FT_THREADS, 0, s>>>(a);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

int launch_flat(const FlatProblem& p, const FlatRole* roles, int n_roles, hipStream_t s) {
  if (p.recv_tokens <= 0 || n_roles <= 0) return KVX_OK;
  FlatKArgs base{};
  base.recv_layers = p.recv_layers;
  base.recv_tokens = p.recv_tokens;
  base.f_in = p.f_in;
  base.f_out = p.f_out;
  base.send_row = p.send_row;
  base.n_taps = p.n_taps;
  base.tab_recv = p.tab_recv;
  base.uniq = p.runs.uniq;
  base.run_begin = p.runs.run_begin;
  base.r2u = p.runs.recv_to_uniq;
  base.n_uniq = p.runs.n_uniq;
  for (int l = 0; l < p.recv_layers; ++l)
    for (int t = 0; t < p.n_taps; ++t)
      base.taps[l * MAX_TAPS + t] = static_cast<uint8_t>(p.taps[l * p.n_taps + t]);

  FlatKArgs& a = base;
  a.n_roles = n_roles;
  for (int j = 0; j < n_roles; ++j) {
    a.a_src[j] = roles[j].a_src;
    a.a_layer_stride[j] = roles[j].a_layer_stride;
    a.a_compact[j] = roles[j].a_compact;
    a.a_f16[j] = roles[j].a_f16;
    a.wt[j] = roles[j].wt;
    a.bias[j] = roles[j].bias;
    a.out[j] = roles[j].out;
    a.rotate[j] = roles[j].rotate;
  }
  return p.w_f32 ? launch_flat_t<2, true>(a, s) : launch_flat_t<1, false>(a, s);
}

}  // namespace kvx
