// Launchers shared between the translation units of the kvx library.
#pragma once

#include "kvx_common.hpp"

namespace kvx {

// Largest layer count a cache may have (layer indices travel as uint8).
constexpr int MAX_LAYERS = 255;
constexpr int MAX_TAPS = 7;

// Zero-fill of int32 words by a kernel (no runtime memset, so the launches of
// a call can be captured into a graph).
int launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// ---------------------------------------------------------------- alignment / runs
size_t align_ws_bytes(int32_t n_recv);
// Several sequences concatenated (host offset arrays of n_seq + 1 entries);
// out holds indices into the concatenated sender tokens.
size_t align_batched_ws_bytes(const int32_t* recv_off, int32_t n_seq);
int launch_align_batched(const int32_t* send_end, const int32_t* send_off, const int32_t* recv_end,
                         const int32_t* recv_off, int32_t n_seq, int32_t* out, void* ws, hipStream_t s);
int launch_align(const int32_t* send_end, int32_t n_send, const int32_t* recv_end,
                 int32_t n_recv, int32_t* out, void* ws, hipStream_t s);

struct Runs {
  int32_t* uniq;          // [N]   value of each run (clamped into [0, n_send))
  int32_t* run_begin;     // [N+1] first row of each run, run_begin[U] = N
  int32_t* recv_to_uniq;  // [N]   run index of each row
  int32_t* n_uniq;        // [1]   U
};
size_t runs_ws_bytes(int32_t n);
int launch_runs(const int32_t* map, int32_t n, int32_t n_send, Runs r, void* ws, hipStream_t s);

// ---------------------------------------------------------------- rotation
// tab[p][j] = (cos, sin)(p * base^(-2j/head_dim)), p < n_pos, j < head_dim/2,
// evaluated in fp64 and rounded to fp32.
int launch_rope_table(float2* tab, int32_t n_pos, int32_t head_dim, double base, hipStream_t s);

// Rotated-back sender keys of the unique rows as fp16:
// out[s][u][h][c] for u < U (device count), every sender layer s with
// layer_used[s] != 0.  Requires head_dim == 128, bf16 cache.
// pos (device [send_tokens], or null = token index): rotary position of each
// sender token, clamped to [0, pos_limit).
int launch_derotate_rows(const uint16_t* k_send, int32_t send_layers, int32_t send_tokens,
                         int32_t heads, const uint8_t* layer_used, const Runs& r,
                         int32_t rows_cap, const float2* tab_send, const int32_t* pos,
                         int32_t pos_limit, uint16_t* out, hipStream_t s);

// ---------------------------------------------------------------- flattened translation
struct FlatRole {
  const void* a_src;       // sender cache (bf16) or rotated-back rows (fp16)
  int64_t a_layer_stride;  // elements between consecutive sender layers of a_src
  int32_t a_compact;       // 1: rows of a_src are run indices u; 0: sender tokens uniq[u]
  int32_t a_f16;           // 1: operands are fp16, 0: bf16
  const void* wt;          // 16-bit map of the operand type, [L_R][F_out][k_dim], or fp8 E4M3 codes
  const float* wscale;     // fp8 maps: [L_R][F_out] scale of each output, else null
  const float* bias;       // [L_R][F_out] or null
  uint16_t* out;           // [L_R][N_R][F_out] bf16
  int32_t rotate;          // rotate outputs at the receiver position
  const float* knorm;      // [L_R][128] key-normalisation weights (before the rotation) or null
};

struct FlatProblem {
  int32_t send_layers, send_tokens, recv_layers, recv_tokens;
  int32_t k_dim;           // n_taps * send_row, doubled for split fp32 maps
  int32_t f_out, n_taps, send_row;  // send_row = H_S * d_S
  const int32_t* taps;     // host [L_R][n_taps]
  const float2* tab_recv;
  Runs runs;
  float knorm_eps;
  const int64_t* slot;     // [N_R] output row of each receiver token, or null (row i)
  int64_t pool_rows;       // output rows per layer
  const int32_t* recv_pos; // [N_R] rotary position of each receiver token, or null (i)
  int32_t pos_limit;       // positions clamped to [0, pos_limit)
  int32_t w8;              // maps are fp8 E4M3 codes with per-output scales
};

int launch_flat(const FlatProblem& p, const FlatRole* roles, int n_roles, hipStream_t s);

// Map preparation: row-major [batch][R][C] (y = x W) -> output-major
// [batch][C][m R] in the kernels' operand type.
enum MapMode : int32_t {
  TM_F32 = 0,        // fp32 -> fp32
  TM_BF16 = 1,       // bf16 -> bf16
  TM_F16 = 2,        // bf16 -> fp16
  TM_SPLIT_BF16 = 3, // fp32 -> [bf16 hi | bf16 lo]  (m = 2)
  TM_SPLIT_F16 = 4,  // fp32 -> [fp16 hi | fp16 lo]  (m = 2)
};
int launch_transpose_maps(const void* in, void* out, int64_t batch, int32_t R, int32_t C, int32_t mode,
                          hipStream_t s);

// fp8 E4M3 quantisation of `count` row-major fp32 maps [f_in][f_out], per
// output o: scale = amax_f |w[f][o]| / 448 (1 for an all-zero output), codes
// = nearest-even E4M3 of w / scale, written output-major q[count][f_out][f_in],
// scale[count][f_out].
int launch_quantize_fp8(const float* w, int64_t count, int32_t f_in, int32_t f_out, uint8_t* q, float* scale,
                        hipStream_t s);

// ---------------------------------------------------------------- per-head translation (bf16)
struct HeadProblem {
  int32_t send_layers, send_tokens, recv_layers, recv_tokens, heads;
  int32_t w_f32;
  const int32_t* taps;         // host [L_R][1]
  const int32_t* recv_to_send;
  const float2* tab_recv;      // receiver RoPE table (rotated roles)
  const int64_t* slot;         // [N_R] output row of each receiver token, or null (row i)
  int64_t pool_rows;           // output rows per layer
  const int32_t* recv_pos;     // [N_R] rotary position of each receiver token, or null (i)
  int32_t pos_limit;
};
struct HeadRole {
  const uint16_t* x;       // sender rows: [L_S][N_S][H][128] bf16, or compact [L_S][rows][H][128] fp16
  int64_t x_layer_stride;  // elements between sender layers of x
  int32_t x_rows;          // rows of one sender layer of x
  const int32_t* row_of;   // [N_R] row of x for each receiver token (the token map, or the run index)
  int32_t x_f16;           // x holds fp16 rows rotated back at the sender position
  int32_t rotate;          // rotate outputs at the receiver position
  const void* wt;          // prepared maps [L_R][H][128 outputs][128 (16-bit) or 2 x 128 (fp32: hi | lo)]
  const float* bias;       // [L_R][H*128] or null
  uint16_t* out;           // [L_R][N_R][H][128]
};
int launch_perhead(const HeadProblem& p, const HeadRole* roles, int n_roles, hipStream_t s);

// ---------------------------------------------------------------- fp32 caches (any shape)
struct F32Problem {
  int32_t send_layers, send_tokens, send_heads, send_dim;
  int32_t recv_layers, recv_tokens, recv_heads, recv_dim;
  int32_t n_taps, per_head, w_f32;
  const int32_t* taps;  // host [L_R][n_taps]
  const int32_t* recv_to_send;
  const float2* tab_send;  // null when the sender keys are unrotated
  const float2* tab_recv;  // null when the receiver keys are unrotated
};
struct F32Role {
  const float* x;
  const void* wt;
  const float* bias;
  float* out;
  int32_t derotate, rotate;
};
int launch_f32(const F32Problem& p, const F32Role* roles, int n_roles, hipStream_t s);

// ---------------------------------------------------------------- fold
// W [f_in][f_out] + A [f_in][rank] B [rank][f_out], per map, row-major.
int launch_fold(const float* w, const float* a, const float* b, int64_t count, int32_t f_in,
                int32_t f_out, int32_t rank, void* out, int32_t out_bf16, hipStream_t s);

// ---------------------------------------------------------------- features / fit
int launch_gather(const void* cache, int32_t cache_f32, int32_t send_tokens, int32_t row,
                  int64_t layer_stride, const int32_t* taps, int32_t n_taps,
                  const int32_t* recv_to_send, int32_t n_rows, double rope_base, int32_t head_dim,
                  void* out, hipStream_t s);

size_t fit_ws_bytes(int32_t count, int32_t f_in, int32_t f_out);
// `count` problems of one shape; x, y, w_out, b_out are host arrays of device
// pointers; status (host, may be null) receives each problem's status.
int launch_fit(int32_t count, const void* const* x, int64_t ldx, const void* const* y, int64_t ldy,
               int32_t in_f32, int64_t n_rows, int32_t f_in, int32_t f_out, double lam_abs,
               double lam_rel, int32_t fit_intercept, float* const* w_out, float* const* b_out,
               int32_t* status, void* ws, hipStream_t s);

// Compute-unit count of the current device (cached per device).
int device_cu_count();

// ---------------------------------------------------------------- measurement probes
// mode 0: copy a -> b; 1: read a (b: sink of probe_read_sink_words() words);
// 2: fill a.  Mean ms per launch over `iters` launches.
int run_probe_hbm(int32_t mode, void* a, void* b, int64_t bytes, int32_t iters, float* ms, hipStream_t s);
int run_probe_mfma(float* out, int32_t reps, int32_t iters, float* ms, double* flops, hipStream_t s);
int probe_mfma_out_floats();
int probe_read_sink_words();

}  // namespace kvx
