// Per-head translation and the fp32-cache translation.
//
// "Cross-Model KV Cache Transfer in Production" (pipeline stage 2) maps each
// KV head with its own d x d matrix when sender and receiver share head count
// and head dimension; stage 3 assigns each receiver layer one sender layer by
// proportional depth.  Several receiver layers may read the same sender layer
// (a deeper receiver), so one block reads a sender tile once and applies the
// maps of every receiver layer assigned to that sender layer.  The work per
// byte is low (a 128 x 128 map per 256-byte row), so this path is bound by
// HBM: X is read once, Y written once, and the fp32 maps are split into a
// bf16 high and low half on the fly (two matrix-core passes keep fp32-level
// accuracy of the map while the bf16 inputs stay exact).

#include "kvx_internal.hpp"

namespace kvx {

// ---------------------------------------------------------------- bf16 caches, d = 128
constexpr int PH_TOK = 256;      // receiver tokens per block (64 per wave)
constexpr int PH_LDW = 136;      // LDS row stride of a staged map (128 + 8)

struct HeadKArgs {
  const uint16_t* x[2];
  const void* wt[2];
  const float* bias[2];
  uint16_t* out[2];
  const int32_t* map;
  int32_t send_layers, send_tokens, recv_layers, recv_tokens, heads, n_chunks;
  int32_t n_blocks, xcd_remap;
  uint8_t first[MAX_LAYERS + 1];   // receiver layers of sender layer s: list[first[s] .. first[s+1])
  uint8_t list[MAX_LAYERS];
};

template <bool WF32>
__global__ __launch_bounds__(256, 2) void perhead_kernel(const HeadKArgs a) {
  constexpr int SPLIT = WF32 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t wsm[SPLIT * 128 * PH_LDW];

  int32_t b = blockIdx.x;
  if (a.xcd_remap) b = (b & 7) * (a.n_blocks >> 3) + (b >> 3);
  const int32_t chunk = b % a.n_chunks;
  int32_t rest = b / a.n_chunks;
  const int32_t h = rest % a.heads;
  rest /= a.heads;
  const int32_t s = rest % a.send_layers;
  const int role = rest / a.send_layers;
  const int32_t l_begin = a.first[s], l_end = a.first[s + 1];
  if (l_begin == l_end) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t tok0 = chunk * PH_TOK + wave * 64;
  const int64_t row_elems = static_cast<int64_t>(a.heads) * 128;

  // X fragments (B operand): token tok0 + 32*ti + lane%32, channels
  // 16*ks + 8*(lane/32) .. +8.
  u32x4 xf[2][8];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    int32_t tok = tok0 + 32 * ti + (lane & 31);
    tok = tok < a.recv_tokens ? tok : a.recv_tokens - 1;
    int32_t src = a.map[tok];
    src = src < 0 ? 0 : (src >= a.send_tokens ? a.send_tokens - 1 : src);
    const uint16_t* xp = a.x[role] + (static_cast<int64_t>(s) * a.send_tokens + src) * row_elems + h * 128 + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) xf[ti][ks] = *reinterpret_cast<const u32x4*>(xp + ks * 16);
  }

  for (int32_t li = l_begin; li < l_end; ++li) {
    const int32_t l = a.list[li];
    __syncthreads();
    // stage W_{l,h} (output-major [o][c]) into LDS as bf16 (hi[, lo])
    if constexpr (WF32) {
      const float* wp = static_cast<const float*>(a.wt[role]) + (static_cast<int64_t>(l) * a.heads + h) * 128 * 128;
#pragma unroll 4
      for (int i = tid; i < 128 * 32; i += 256) {
        const int o = i >> 5, c4 = (i & 31) * 4;
        const float4 v = *reinterpret_cast<const float4*>(wp + o * 128 + c4);
        const uint32_t h0 = pack_bf16(v.x, v.y), h1 = pack_bf16(v.z, v.w);
        const uint32_t l0 = pack_bf16(v.x - bf16lo(h0), v.y - bf16hi(h0));
        const uint32_t l1 = pack_bf16(v.z - bf16lo(h1), v.w - bf16hi(h1));
        *reinterpret_cast<u32x2*>(wsm + o * PH_LDW + c4) = u32x2{h0, h1};
        *reinterpret_cast<u32x2*>(wsm + 128 * PH_LDW + o * PH_LDW + c4) = u32x2{l0, l1};
      }
    } else {
      const uint16_t* wp = static_cast<const uint16_t*>(a.wt[role]) + (static_cast<int64_t>(l) * a.heads + h) * 128 * 128;
#pragma unroll 4
      for (int i = tid; i < 128 * 16; i += 256) {
        const int o = i >> 4, c8 = (i & 15) * 8;
        *reinterpret_cast<u32x4*>(wsm + o * PH_LDW + c8) = *reinterpret_cast<const u32x4*>(wp + o * 128 + c8);
      }
    }
    __syncthreads();

    f32x16 acc[2][4];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[ti][ni][e] = 0.0f;

#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
        for (int sp = 0; sp < SPLIT; ++sp) {
          const u32x4 wf = *reinterpret_cast<const u32x4*>(
              wsm + sp * 128 * PH_LDW + (ni * 32 + (lane & 31)) * PH_LDW + ks * 16 + (lane >> 5) * 8);
#pragma unroll
          for (int ti = 0; ti < 2; ++ti)
            acc[ti][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, wf), __builtin_bit_cast(bf16x8, xf[ti][ks]), acc[ti][ni], 0, 0, 0);
        }
      }
    }

    // D[n][tok]: lane holds token 32*ti + lane%32 and outputs
    // n = 32*ni + 8*(r/4) + 4*(lane/32) + r%4.
    const float* bias = a.bias[role] ? a.bias[role] + static_cast<int64_t>(l) * row_elems + h * 128 : nullptr;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const int32_t tok = tok0 + 32 * ti + (lane & 31);
      if (tok >= a.recv_tokens) continue;
      uint16_t* op = a.out[role] + (static_cast<int64_t>(l) * a.recv_tokens + tok) * row_elems + h * 128;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = ni * 32 + 8 * g + 4 * (lane >> 5);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[ti][ni][4 * g + e] + (bias ? bias[n + e] : 0.0f);
          *reinterpret_cast<u32x2*>(op + n) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        }
    }
  }
}

int launch_perhead(const HeadProblem& p, const HeadRole* roles, int n_roles, hipStream_t s) {
  if (p.recv_tokens <= 0 || n_roles <= 0) return KVX_OK;
  HeadKArgs a{};
  for (int i = 0; i < n_roles; ++i) {
    a.x[i] = roles[i].x;
    a.wt[i] = roles[i].wt;
    a.bias[i] = roles[i].bias;
    a.out[i] = roles[i].out;
  }
  a.map = p.recv_to_send;
  a.send_layers = p.send_layers;
  a.send_tokens = p.send_tokens;
  a.recv_layers = p.recv_layers;
  a.recv_tokens = p.recv_tokens;
  a.heads = p.heads;
  a.n_chunks = static_cast<int32_t>(ceil_div(p.recv_tokens, PH_TOK));
  // receiver layers grouped by their sender layer (counting sort, ascending l)
  int cnt[MAX_LAYERS + 1] = {0};
  for (int l = 0; l < p.recv_layers; ++l) cnt[p.taps[l] + 1]++;
  for (int q = 0; q < p.send_layers; ++q) cnt[q + 1] += cnt[q];
  for (int q = 0; q <= p.send_layers; ++q) a.first[q] = static_cast<uint8_t>(cnt[q]);
  int fill[MAX_LAYERS] = {0};
  for (int l = 0; l < p.recv_layers; ++l) {
    const int q = p.taps[l];
    a.list[cnt[q] + fill[q]++] = static_cast<uint8_t>(l);
  }
  const int64_t nb = static_cast<int64_t>(n_roles) * p.send_layers * p.heads * a.n_chunks;
  a.n_blocks = static_cast<int32_t>(nb);
  a.xcd_remap = (nb % 8 == 0) ? 1 : 0;
  if (p.w_f32)
    perhead_kernel<true><<<static_cast<unsigned>(nb), 256, 0, s>>>(a);
  else
    perhead_kernel<false><<<static_cast<unsigned>(nb), 256, 0, s>>>(a);
  KVX_LAUNCH_CHECK();
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
