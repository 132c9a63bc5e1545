// Rotary position handling and feature gathers.
//
// "Cross-Model KV Cache Transfer in Production" (pipeline stage 1) strips the
// sender's rotation from cached keys, K_content = R_{-m} K_m, and stage 4
// applies the receiver's own rotation at the receiver position; values are
// never rotated.  The rotation acts on half-split pairs (c, c + d/2) with
// angle pos * base^(-2j/d) for pair j.  Angles reach tens of thousands of
// radians at long context, so they are formed in fp64 here (a sincos per run
// of positions, fp64 angle-addition steps inside the run) and kept as an
// fp32 (cos, sin) table.

#include "kvx_internal.hpp"

namespace kvx {

// One thread: frequency j (consecutive lanes take consecutive j, so the
// stores of a position are one contiguous row) for RT_RUN consecutive
// positions p0 .. p0 + RT_RUN - 1.  theta_j = base^(-2j/head_dim) in fp64;
// (cos, sin)(p0 theta) from fp64 sincos, then each next position by the fp64
// angle-addition step (cos, sin)((p+1) theta) = (c cos(theta) - s sin(theta),
// s cos(theta) + c sin(theta)); over RT_RUN steps the fp64 recurrence drifts
// by ~1e-14, far below the fp32 rounding of the stored table.
constexpr int RT_RUN = 32;
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ tab, int32_t n_pos, int32_t half,
                                                         int32_t head_dim, double base) {
  const int64_t runs = (static_cast<int64_t>(n_pos) + RT_RUN - 1) / RT_RUN;
  const int64_t total = runs * half;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int32_t j = static_cast<int32_t>(i % half);
    const int32_t p0 = static_cast<int32_t>(i / half) * RT_RUN;
    const double theta = pow(base, -2.0 * static_cast<double>(j) / static_cast<double>(head_dim));
    double s, c, st, ct;
    sincos(static_cast<double>(p0) * theta, &s, &c);
    sincos(theta, &st, &ct);
    const int32_t n = min(RT_RUN, n_pos - p0);
    for (int32_t r = 0; r < n; ++r) {
      tab[static_cast<int64_t>(p0 + r) * half + j] = make_float2(static_cast<float>(c), static_cast<float>(s));
      const double cn = c * ct - s * st;
      s = s * ct + c * st;
      c = cn;
    }
  }
}

int launch_rope_table(float2* tab, int32_t n_pos, int32_t head_dim, double base, hipStream_t s) {
  const int32_t half = head_dim / 2;
  const int64_t total = (static_cast<int64_t>(n_pos) + RT_RUN - 1) / RT_RUN * half;
  if (total <= 0) return KVX_OK;
  int64_t blocks = ceil_div(total, 256);
  if (blocks > 8192) blocks = 8192;
  rope_table_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(tab, n_pos, half, head_dim, base);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// ---------------------------------------------------------------- rotated-back unique rows
// One thread: 8 pairs (j .. j+7 and j+64 .. j+71) of one head of one row.
// Block: 16 rows of one sender layer (blockIdx.y indexes the used layers).
constexpr int DR_ROWS = 16;

struct LayerList {
  uint8_t l[MAX_LAYERS];
};

__global__ __launch_bounds__(256) void derotate_rows_kernel(
    const uint16_t* __restrict__ k_send, int32_t send_tokens, int32_t heads, const int32_t* __restrict__ uniq,
    const int32_t* __restrict__ n_uniq, int32_t rows_cap, const float2* __restrict__ tab,
    const int32_t* __restrict__ pos, int32_t pos_limit, uint16_t* __restrict__ out, const LayerList layers) {
  const int32_t U = min(*n_uniq, rows_cap);
  const int32_t row0 = blockIdx.x * DR_ROWS;
  if (row0 >= U) return;
  const int32_t layer = layers.l[blockIdx.y];
  const int32_t row_elems = heads * 128;
  const int32_t per_row = heads * 8;  // threads per row
  for (int32_t it = threadIdx.x; it < DR_ROWS * per_row; it += 256) {
    const int32_t u = row0 + it / per_row;
    if (u >= U) break;
    const int32_t h = (it % per_row) / 8;
    const int32_t q = it % 8;
    const int32_t p = uniq[u];
    const uint16_t* src = k_send + (static_cast<int64_t>(layer) * send_tokens + p) * row_elems + h * 128;
    const u32x4 a = *reinterpret_cast<const u32x4*>(src + 8 * q);
    const u32x4 b = *reinterpret_cast<const u32x4*>(src + 64 + 8 * q);
    int32_t pp = p;  // rotary position of the sender token
    if (pos) {
      pp = pos[p];
      pp = pp < 0 ? 0 : (pp >= pos_limit ? pos_limit - 1 : pp);
    }
    const float4* t4 = reinterpret_cast<const float4*>(tab + static_cast<int64_t>(pp) * 64 + 8 * q);
    uint32_t oa[4], ob[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 cs = t4[w];  // (cos, sin) of pairs 2w and 2w+1
      const float a0 = bf16lo(a[w]), a1 = bf16hi(a[w]);
      const float b0 = bf16lo(b[w]), b1 = bf16hi(b[w]);
      // rotation by -angle: (a, b) -> (a cos + b sin, -a sin + b cos)
      const float ra0 = a0 * cs.x + b0 * cs.y, rb0 = b0 * cs.x - a0 * cs.y;
      const float ra1 = a1 * cs.z + b1 * cs.w, rb1 = b1 * cs.z - a1 * cs.w;
      oa[w] = pack_f16(ra0, ra1);
      ob[w] = pack_f16(rb0, rb1);
    }
    uint16_t* dst = out + (static_cast<int64_t>(layer) * rows_cap + u) * row_elems + h * 128;
    *reinterpret_cast<u32x4*>(dst + 8 * q) = u32x4{oa[0], oa[1], oa[2], oa[3]};
    *reinterpret_cast<u32x4*>(dst + 64 + 8 * q) = u32x4{ob[0], ob[1], ob[2], ob[3]};
  }
}

int launch_derotate_rows(const uint16_t* k_send, int32_t send_layers, int32_t send_tokens, int32_t heads,
                         const uint8_t* layer_used, const Runs& r, int32_t rows_cap, const float2* tab_send,
                         const int32_t* pos, int32_t pos_limit, uint16_t* out, hipStream_t s) {
  if (rows_cap <= 0) return KVX_OK;
  LayerList ll{};
  int n = 0;
  for (int32_t l = 0; l < send_layers; ++l)
    if (layer_used[l]) ll.l[n++] = static_cast<uint8_t>(l);
  if (n == 0) return KVX_OK;
  const dim3 grid(static_cast<unsigned>(ceil_div(rows_cap, DR_ROWS)), static_cast<unsigned>(n));
  derotate_rows_kernel<<<grid, 256, 0, s>>>(k_send, send_tokens, heads, r.uniq, r.n_uniq, rows_cap, tab_send, pos,
                                            pos_limit, out, ll);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// ---------------------------------------------------------------- feature gather
// out[i][t*row + e] = cache[taps[t]][map[i]][e], keys optionally rotated back
// at position map[i] (angle formed and reduced in fp64 per pair; this gather
// materialises fit inputs once, so no table is kept).  One thread: one pair
// (c, c + d/2) of a head when rotating, else two neighbouring elements.
struct GatherTaps {
  int32_t t[MAX_TAPS];
};

template <bool F32>
__global__ __launch_bounds__(256) void gather_kernel(
    const void* __restrict__ cache, int32_t send_tokens, int32_t row, int64_t layer_stride,
    GatherTaps taps, int32_t n_taps, const int32_t* __restrict__ map, int32_t n_rows,
    double rope_base, int32_t head_dim, void* __restrict__ out) {
  const int32_t i = blockIdx.x;
  if (i >= n_rows) return;
  int32_t p = map[i];
  p = p < 0 ? 0 : (p >= send_tokens ? send_tokens - 1 : p);
  const int32_t half = head_dim / 2;
  const int32_t n_pairs = row / 2;
  const int64_t f_in = static_cast<int64_t>(n_taps) * row;
  const bool rot = rope_base > 0.0;
  for (int32_t t = 0; t < n_taps; ++t) {
    const int64_t src_off = static_cast<int64_t>(taps.t[t]) * layer_stride + static_cast<int64_t>(p) * row;
    for (int32_t k = threadIdx.x; k < n_pairs; k += blockDim.x) {
      int32_t e0, e1;
      if (rot) {
        const int32_t h = k / half, j = k % half;
        e0 = h * head_dim + j;
        e1 = e0 + half;
      } else {
        e0 = 2 * k;
        e1 = e0 + 1;
      }
      float a, b;
      if (F32) {
        const float* c = static_cast<const float*>(cache) + src_off;
        a = c[e0];
        b = c[e1];
      } else {
        const uint16_t* c = static_cast<const uint16_t*>(cache) + src_off;
        a = bf16_to_f32(c[e0]);
        b = bf16_to_f32(c[e1]);
      }
      if (rot) {
        const double theta = pow(rope_base, -2.0 * static_cast<double>(k % half) / static_cast<double>(head_dim));
        double sn, cs;
        sincos(static_cast<double>(p) * theta, &sn, &cs);
        const float c32 = static_cast<float>(cs), s32 = static_cast<float>(sn);
        const float ra = a * c32 + b * s32;
        const float rb = b * c32 - a * s32;
        a = ra;
        b = rb;
      }
      const int64_t o = static_cast<int64_t>(i) * f_in + static_cast<int64_t>(t) * row;
      if (F32) {
        float* dst = static_cast<float*>(out) + o;
        dst[e0] = a;
        dst[e1] = b;
      } else {
        uint16_t* dst = static_cast<uint16_t*>(out) + o;
        dst[e0] = f32_to_bf16_rne(a);
        dst[e1] = f32_to_bf16_rne(b);
      }
    }
  }
}

int launch_gather(const void* cache, int32_t cache_f32, int32_t send_tokens, int32_t row,
                  int64_t layer_stride, const int32_t* taps, int32_t n_taps,
                  const int32_t* recv_to_send, int32_t n_rows, double rope_base, int32_t head_dim,
                  void* out, hipStream_t s) {
  if (n_rows <= 0) return KVX_OK;
  GatherTaps gt{};
  for (int t = 0; t < n_taps; ++t) gt.t[t] = taps[t];
  if (cache_f32)
    gather_kernel<true><<<n_rows, 256, 0, s>>>(cache, send_tokens, row, layer_stride, gt, n_taps,
                                               recv_to_send, n_rows, rope_base, head_dim, out);
  else
    gather_kernel<false><<<n_rows, 256, 0, s>>>(cache, send_tokens, row, layer_stride, gt, n_taps,
                                                recv_to_send, n_rows, rope_base, head_dim, out);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

// ---------------------------------------------------------------- rank-r fold
// "Prefill-Free ...", Methodology 3: the rank-16 corrections are folded into
// one fixed map, W_eff = W + A B with W [f_in][f_out], A [f_in][rank],
// B [rank][f_out] (row-major, y = x W).  Products rounded to fp32, summed in
// rank order, added to the dense entry, then stored (bf16: nearest even).
// Contraction into fused multiply-adds is switched off so the order of
// roundings is the stated one.  One thread per entry (f, o); consecutive
// threads take consecutive o, so the reads of W and B and the writes run
// along rows.
__global__ __launch_bounds__(256) void fold_kernel(const float* __restrict__ w,
                                                   const float* __restrict__ a,
                                                   const float* __restrict__ b, int64_t count,
                                                   int32_t f_in, int32_t f_out, int32_t rank,
                                                   void* __restrict__ out, int32_t out_bf16) {
#pragma clang fp contract(off)
  const int64_t per = static_cast<int64_t>(f_in) * f_out;
  const int64_t total = per * count;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t m = i / per;
    const int64_t r0 = i % per;
    const int32_t f = static_cast<int32_t>(r0 / f_out);
    const int32_t o = static_cast<int32_t>(r0 % f_out);
    const float* ar = a + (m * f_in + f) * rank;
    const float* bc = b + m * rank * static_cast<int64_t>(f_out) + o;
    float acc = 0.0f;
    for (int32_t r = 0; r < rank; ++r) {
      const float p = ar[r] * bc[static_cast<int64_t>(r) * f_out];
      acc = (r == 0) ? p : acc + p;
    }
    const float tot = (rank > 0) ? w[i] + acc : w[i];
    if (out_bf16)
      static_cast<uint16_t*>(out)[i] = f32_to_bf16_rne(tot);
    else
      static_cast<float*>(out)[i] = tot;
  }
}

int launch_fold(const float* w, const float* a, const float* b, int64_t count, int32_t f_in,
                int32_t f_out, int32_t rank, void* out, int32_t out_bf16, hipStream_t s) {
  const int64_t total = count * f_in * static_cast<int64_t>(f_out);
  if (total <= 0) return KVX_OK;
  int64_t blocks = ceil_div(total, 256);
  if (blocks > 65536) blocks = 65536;
  fold_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(w, a, b, count, f_in, f_out, rank, out,
                                                            out_bf16);
  KVX_LAUNCH_CHECK();
  return KVX_OK;
}

}  // namespace kvx
