// C-ABI entry points of the kvx library: argument validation, workspace
// layout and kernel launch order.  Every computation runs in the HIP kernels
// of the other translation units; this file only checks shapes and wires
// buffers.

#include <mutex>

#include "kvx_fit.hpp"
#include "kvx_align.hpp"

namespace kvx {

constexpr int32_t RECV_TAB_MIN = 16;
static int32_t recv_tab_rows(int32_t n) { return n > RECV_TAB_MIN ? n : RECV_TAB_MIN; }

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> g(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static bool desc_ok(const kvx_cache_desc* d) {
  if (!d) return false;
  if (d->layers < 1 || d->layers > MAX_LAYERS || d->tokens < 0 || d->kv_heads < 1 || d->head_dim < 1) return false;
  if (static_cast<int64_t>(d->kv_heads) * d->head_dim > KVX_MAX_ROW) return false;
  if (d->dtype != KVX_F32 && d->dtype != KVX_BF16) return false;
  if (!(d->rope_base >= 0.0)) return false;
  if (d->rope_base > 0.0 && (d->head_dim % 2) != 0) return false;
  if (d->k_norm && !(d->k_norm_eps >= 0.0)) return false;
  return true;
}

// Kernel layout of one role's maps (what kvx_prepare_maps writes): the
// caller's row-major [batch][R][C] maps transposed to output-major in the
// operand type of the path that reads them.
struct MapFormat {
  int32_t mode = TM_F32;
  int64_t batch = 0;
  int32_t R = 0, C = 0;
  size_t bytes = 0;
};

static MapFormat map_format(const kvx_cache_desc* send, const kvx_cache_desc* recv, int32_t n_taps,
                            int32_t per_head, bool key_role, int32_t w_dtype) {
  MapFormat f;
  const bool wf32 = w_dtype == KVX_F32;
  if (per_head) {
    f.batch = static_cast<int64_t>(recv->layers) * recv->kv_heads;
    f.R = f.C = recv->head_dim;
  } else {
    f.batch = recv->layers;
    f.R = n_taps * send->kv_heads * send->head_dim;
    f.C = recv->kv_heads * recv->head_dim;
  }
  const size_t elems = static_cast<size_t>(f.batch) * f.R * f.C;
  if (send->dtype == KVX_F32) {
    // fp32 caches: the map in its own type
    f.mode = wf32 ? TM_F32 : TM_BF16;
    f.bytes = elems * (wf32 ? 4 : 2);
  } else {
    // bf16 caches (flattened and per head): 16-bit operands of the role's
    // type (fp16 for keys rotated back from a rotated sender), fp32 maps
    // split in two
    const bool f16 = key_role && send->rope_base > 0.0;
    if (wf32) {
      f.mode = f16 ? TM_SPLIT_F16 : TM_SPLIT_BF16;
      f.bytes = elems * 4;
    } else {
      f.mode = f16 ? TM_F16 : TM_BF16;
      f.bytes = elems * 2;
    }
  }
  return f;
}

// Workspace layout of kvx_translate.  Returned sizes and the slices used by
// the launch come from this single function.
struct TranslateWs {
  Runs runs{};
  void* runs_scratch = nullptr;
  float2* tab_send = nullptr;
  float2* tab_recv = nullptr;
  uint16_t* krows = nullptr;   // rotated-back unique key rows (fp16)
  void* wk = nullptr;          // key maps in the kernel layout (raw calls)
  void* wv = nullptr;          // value maps in the kernel layout (raw calls)
  int32_t rows_cap = 0;
  size_t bytes = 0;
};

// Rows of the rotation tables: positions 0 .. rows-1.
static int32_t send_tab_rows(const kvx_cache_desc* send, int32_t pos_limit) {
  return send->tokens > pos_limit ? send->tokens : pos_limit;
}
static int32_t recv_tab_rows_for(const kvx_cache_desc* recv, int32_t pos_limit) {
  const int32_t r = recv_tab_rows(recv->tokens);
  return r > pos_limit ? r : pos_limit;
}

// map element type of the fp8 entry point (internal; not a kvx_dtype)
constexpr int32_t W_FP8 = 2;

// raw: the maps arrive in the caller's layout and are prepared into the
// workspace (sized for w_dtype).
static TranslateWs layout_translate(const kvx_cache_desc* send, const kvx_cache_desc* recv, int32_t n_taps,
                                    int32_t per_head, int32_t w_dtype, bool key_role, bool value_role,
                                    int32_t pos_limit, bool raw, void* base) {
  TranslateWs w;
  Carve c(base);
  const int32_t nr = recv->tokens;
  const bool f32 = send->dtype == KVX_F32;
  const bool srope = send->rope_base > 0.0 && key_role;
  const bool rrope = recv->rope_base > 0.0 && key_role;
  // runs of equal sender tokens: the flattened path's row index, and the
  // index of rotated-back key rows on both paths
  if (!f32 && (!per_head || srope)) {
    w.runs.uniq = c.take<int32_t>(nr > 0 ? nr : 1);
    w.runs.run_begin = c.take<int32_t>(static_cast<size_t>(nr) + 1);
    w.runs.recv_to_uniq = c.take<int32_t>(nr > 0 ? nr : 1);
    w.runs.n_uniq = c.take<int32_t>(64);
    w.runs_scratch = c.take<char>(runs_ws_bytes(nr));
  }
  if (srope) w.tab_send = c.take<float2>(static_cast<size_t>(send_tab_rows(send, pos_limit)) * (send->head_dim / 2));
  // the receiver table holds at least RECV_TAB_MIN positions: the flattened
  // epilogue reads the (cos, sin) step of its rotation recurrence from the
  // table row of position 8, also for caches of fewer tokens
  if (rrope) w.tab_recv = c.take<float2>(static_cast<size_t>(recv_tab_rows_for(recv, pos_limit)) * (recv->head_dim / 2));
  if (!f32 && srope) {
    // U <= N_R always (U <= N_S only for non-decreasing maps)
    w.rows_cap = nr;
    w.krows = c.take<uint16_t>(static_cast<size_t>(send->layers) * w.rows_cap * send->kv_heads * send->head_dim);
  }
  if (raw && w_dtype != W_FP8) {
    if (key_role) w.wk = c.take<char>(map_format(send, recv, n_taps, per_head, true, w_dtype).bytes);
    if (value_role) w.wv = c.take<char>(map_format(send, recv, n_taps, per_head, false, w_dtype).bytes);
  }
  w.bytes = c.used + 256;
  return w;
}

}  // namespace kvx

using namespace kvx;

static_assert(KVX_NOALLOC_MAX_RECV == NOALLOC_MAX_RECV, "header and library limits of the no-allocation alignment");

extern "C" {

const char* kvx_status_string(int status) {
  switch (status) {
    case KVX_OK: return "ok";
    case KVX_ERR_INVALID: return "invalid argument";
    case KVX_ERR_SHAPE: return "inconsistent shapes";
    case KVX_ERR_WORKSPACE: return "workspace missing or too small";
    case KVX_ERR_NOT_SPD: return "regularised Gram matrix is not positive definite";
    case KVX_ERR_HIP: return "HIP runtime error";
    case KVX_ERR_UNSUPPORTED: return "unsupported combination";
    case KVX_ERR_NOT_CONVERGED: return "iteration did not converge";
    default: return "unknown status";
  }
}

size_t kvx_align_workspace_size(int32_t n_recv) { return align_ws_bytes(n_recv) + 256; }

int kvx_align_tokens(const int32_t* send_end, int32_t n_send, const int32_t* recv_end, int32_t n_recv,
                     int32_t* recv_to_send, void* workspace, size_t ws_bytes, void* stream) {
  if (n_send < 0 || n_recv < 0) return KVX_ERR_INVALID;
  if (n_recv == 0) return KVX_OK;
  if (n_send == 0) return KVX_ERR_SHAPE;
  if (!send_end || !recv_end || !recv_to_send) return KVX_ERR_INVALID;
  if (!workspace || ws_bytes < kvx_align_workspace_size(n_recv)) return KVX_ERR_WORKSPACE;
  return launch_align(send_end, n_send, recv_end, n_recv, recv_to_send, workspace,
                      static_cast<hipStream_t>(stream));
}

int kvx_align_tokens_async(const int32_t* send_end, int32_t n_send, const int32_t* recv_end, int32_t n_recv,
                           int32_t* recv_to_send, int32_t* invalid, void* workspace, size_t ws_bytes, void* stream) {
  if (n_send < 0 || n_recv < 0) return KVX_ERR_INVALID;
  if (n_recv == 0) return KVX_OK;
  if (n_send == 0) return KVX_ERR_SHAPE;
  if (!send_end || !recv_end || !recv_to_send || !invalid) return KVX_ERR_INVALID;
  if (!workspace || ws_bytes < kvx_align_workspace_size(n_recv)) return KVX_ERR_WORKSPACE;
  return launch_align_async(send_end, n_send, recv_end, n_recv, recv_to_send, invalid, workspace,
                            static_cast<hipStream_t>(stream));
}

int kvx_align_tokens_noalloc(const int32_t* send_end, int32_t n_send, const int32_t* recv_end, int32_t n_recv,
                             int32_t* recv_to_send, int32_t* invalid, void* stream) {
  if (n_send < 0 || n_recv < 0) return KVX_ERR_INVALID;
  if (n_recv > KVX_NOALLOC_MAX_RECV) return KVX_ERR_WORKSPACE;
  if (n_recv == 0) return KVX_OK;
  if (n_send == 0) return KVX_ERR_SHAPE;
  if (!send_end || !recv_end || !recv_to_send || !invalid) return KVX_ERR_INVALID;
  return launch_align_noalloc(send_end, n_send, recv_end, n_recv, recv_to_send, invalid,
                              static_cast<hipStream_t>(stream));
}

size_t kvx_align_batched_workspace_size(const int32_t* recv_off, int32_t n_seq) {
  if (!recv_off || n_seq < 1 || recv_off[0] != 0) return 0;
  for (int32_t q = 0; q < n_seq; ++q)
    if (recv_off[q + 1] < recv_off[q]) return 0;
  return align_batched_ws_bytes(recv_off, n_seq) + 256;
}

int kvx_align_tokens_batched(const int32_t* send_end, const int32_t* send_off, const int32_t* recv_end,
                             const int32_t* recv_off, int32_t n_seq, int32_t* recv_to_send, void* workspace,
                             size_t ws_bytes, void* stream) {
  if (n_seq < 1 || !send_off || !recv_off) return KVX_ERR_INVALID;
  if (send_off[0] != 0 || recv_off[0] != 0) return KVX_ERR_INVALID;
  for (int32_t q = 0; q < n_seq; ++q) {
    if (send_off[q + 1] < send_off[q] || recv_off[q + 1] < recv_off[q]) return KVX_ERR_INVALID;
    if (recv_off[q + 1] > recv_off[q] && send_off[q + 1] == send_off[q]) return KVX_ERR_SHAPE;
  }
  if (recv_off[n_seq] == 0) return KVX_OK;
  if (!send_end || !recv_end || !recv_to_send) return KVX_ERR_INVALID;
  if (!workspace || ws_bytes < kvx_align_batched_workspace_size(recv_off, n_seq)) return KVX_ERR_WORKSPACE;
  return launch_align_batched(send_end, send_off, recv_end, recv_off, n_seq, recv_to_send, workspace,
                              static_cast<hipStream_t>(stream));
}

int kvx_layer_map(int32_t send_layers, int32_t recv_layers, int32_t n_taps, int32_t tap_stride, int32_t* taps_out) {
  if (send_layers < 1 || recv_layers < 1 || !taps_out) return KVX_ERR_INVALID;
  if (n_taps < 1 || n_taps > MAX_TAPS || (n_taps % 2) == 0 || tap_stride < 0) return KVX_ERR_INVALID;
  for (int32_t l = 0; l < recv_layers; ++l) {
    int64_t m = 0;
    if (recv_layers > 1) {
      // round(l (L_S-1) / (L_R-1)), halves up, in integers
      const int64_t num = 2LL * l * (send_layers - 1) + (recv_layers - 1);
      m = num / (2LL * (recv_layers - 1));
    }
    for (int32_t t = 0; t < n_taps; ++t) {
      int64_t v = m + static_cast<int64_t>(t - (n_taps - 1) / 2) * tap_stride;
      v = v < 0 ? 0 : (v > send_layers - 1 ? send_layers - 1 : v);
      taps_out[l * n_taps + t] = static_cast<int32_t>(v);
    }
  }
  return KVX_OK;
}

size_t kvx_translate_workspace_size(const kvx_cache_desc* send, const kvx_cache_desc* recv, int32_t n_taps,
                                    int32_t per_head) {
  if (!desc_ok(send) || !desc_ok(recv) || n_taps < 1 || n_taps > MAX_TAPS) return 0;
  // sized for fp32 maps (the larger case) and both roles
  return layout_translate(send, recv, n_taps, per_head, KVX_F32, true, true, 0, true, nullptr).bytes;
}

size_t kvx_translate_prepared_workspace_size(const kvx_cache_desc* send, const kvx_cache_desc* recv,
                                             int32_t n_taps, int32_t per_head, int32_t pos_limit) {
  if (!desc_ok(send) || !desc_ok(recv) || n_taps < 1 || n_taps > MAX_TAPS || pos_limit < 0) return 0;
  return layout_translate(send, recv, n_taps, per_head, KVX_F32, true, true, pos_limit, false, nullptr).bytes;
}

size_t kvx_prepared_maps_size(const kvx_cache_desc* send, const kvx_cache_desc* recv, int32_t n_taps,
                              int32_t per_head, int32_t role, int32_t w_dtype) {
  if (!desc_ok(send) || !desc_ok(recv) || n_taps < 1 || n_taps > MAX_TAPS) return 0;
  if ((role != 0 && role != 1) || (w_dtype != KVX_F32 && w_dtype != KVX_BF16)) return 0;
  return map_format(send, recv, per_head ? 1 : n_taps, per_head, role == 0, w_dtype).bytes;
}

int kvx_prepare_maps(const kvx_cache_desc* send, const kvx_cache_desc* recv, int32_t n_taps, int32_t per_head,
                     int32_t role, int32_t w_dtype, const void* w, void* prepared, size_t prepared_bytes,
                     void* stream) {
  if (!desc_ok(send) || !desc_ok(recv) || n_taps < 1 || n_taps > MAX_TAPS) return KVX_ERR_INVALID;
  if ((role != 0 && role != 1) || (w_dtype != KVX_F32 && w_dtype != KVX_BF16)) return KVX_ERR_INVALID;
  if (per_head && (n_taps != 1 || send->kv_heads != recv->kv_heads || send->head_dim != recv->head_dim))
    return KVX_ERR_SHAPE;
  if (!w || !prepared) return KVX_ERR_INVALID;
  const MapFormat f = map_format(send, recv, n_taps, per_head, role == 0, w_dtype);
  if (prepared_bytes < f.bytes) return KVX_ERR_WORKSPACE;
  return launch_transpose_maps(w, prepared, f.batch, f.R, f.C, f.mode, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace kvx {

// Records ev[0] before the preparation kernels, ev[1] before the main
// translation kernel and ev[2] after it, when ev is not null.  raw: the maps
// wt_k, wt_v are the caller's row-major maps and are put into the kernel
// layout in the workspace first; otherwise they are already in it (prepared
// maps, or fp8 codes).
static int translate_impl(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                          const kvx_cache_desc* recv, void* k_recv, void* v_recv, const int32_t* recv_to_send,
                          const int32_t* taps, int32_t n_taps, int32_t per_head, int32_t w_dtype, const void* wt_k,
                          const void* wt_v, const float* b_k, const float* b_v, void* workspace, size_t ws_bytes,
                          void* stream, hipEvent_t* ev, const kvx_placement* pl, bool raw,
                          const float* s_k = nullptr, const float* s_v = nullptr) {
  if (!desc_ok(send) || !desc_ok(recv)) return KVX_ERR_INVALID;
  if (w_dtype != KVX_F32 && w_dtype != KVX_BF16 && w_dtype != W_FP8) return KVX_ERR_INVALID;
  if (w_dtype == W_FP8) {
    // fp8 maps: flattened matrix-core path, scales of every present role
    if ((k_recv && !s_k) || (v_recv && !s_v)) return KVX_ERR_INVALID;
    if (per_head || send->dtype != KVX_BF16) return KVX_ERR_UNSUPPORTED;
  }
  if (n_taps < 1 || n_taps > MAX_TAPS || !taps) return KVX_ERR_INVALID;
  const bool do_k = k_recv != nullptr, do_v = v_recv != nullptr;
  if (do_k && (!k_send || !wt_k)) return KVX_ERR_INVALID;
  if (do_v && (!v_send || !wt_v)) return KVX_ERR_INVALID;
  if (recv->tokens > 0 && !recv_to_send) return KVX_ERR_INVALID;
  for (int32_t i = 0; i < recv->layers * n_taps; ++i)
    if (taps[i] < 0 || taps[i] >= send->layers) return KVX_ERR_INVALID;
  if (per_head) {
    if (n_taps != 1) return KVX_ERR_SHAPE;
    if (send->kv_heads != recv->kv_heads || send->head_dim != recv->head_dim) return KVX_ERR_SHAPE;
  }
  if (send->dtype != recv->dtype) return KVX_ERR_UNSUPPORTED;
  // placement into a pool of rows, per-token rotary positions
  const int64_t* slot = pl ? pl->slot : nullptr;
  const int32_t* recv_pos = pl ? pl->recv_pos : nullptr;
  const int32_t* send_pos = pl ? pl->send_pos : nullptr;
  const int32_t pos_limit = (recv_pos || send_pos) ? pl->pos_limit : 0;
  int64_t pool_rows = recv->tokens;
  if (pl) {
    if (pl->pool_rows < 0 || (slot && pl->pool_rows < 1)) return KVX_ERR_INVALID;
    if (!slot && pl->pool_rows != 0 && pl->pool_rows < recv->tokens) return KVX_ERR_SHAPE;
    if (pl->pool_rows != 0) pool_rows = pl->pool_rows;
    if ((recv_pos || send_pos) && pl->pos_limit < 1) return KVX_ERR_INVALID;
    if ((slot || recv_pos || send_pos || pool_rows != recv->tokens) && send->dtype == KVX_F32)
      return KVX_ERR_UNSUPPORTED;
  }
  // the receiver's key normalisation: flattened bf16 path (one head of
  // 128 outputs per wave in the epilogue)
  if (recv->k_norm && do_k && (per_head || send->dtype != KVX_BF16)) return KVX_ERR_UNSUPPORTED;
  if (recv->tokens == 0 || (!do_k && !do_v)) return KVX_OK;
  if (send->tokens == 0) return KVX_ERR_SHAPE;
  const bool raw_maps = raw && w_dtype != W_FP8;
  const TranslateWs need =
      layout_translate(send, recv, n_taps, per_head, KVX_F32, true, true, pos_limit, raw_maps, nullptr);
  if (!workspace || ws_bytes < need.bytes) return KVX_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const TranslateWs w =
      layout_translate(send, recv, n_taps, per_head, w_dtype, do_k, do_v, pos_limit, raw_maps, workspace);
  auto mark = [&](int i) -> int {
    if (ev && hipEventRecord(ev[i], s) != hipSuccess) return KVX_ERR_HIP;
    return KVX_OK;
  };
  auto main_kernel = [&](auto&& launch) -> int {
    if (int st = mark(1)) return st;
    if (int st = launch()) return st;
    return mark(2);
  };
  if (int st = mark(0)) return st;
  if (raw_maps) {
    // the caller's row-major maps into the kernel layout
    if (do_k) {
      const MapFormat f = map_format(send, recv, n_taps, per_head, true, w_dtype);
      if (int st = launch_transpose_maps(wt_k, w.wk, f.batch, f.R, f.C, f.mode, s)) return st;
      wt_k = w.wk;
    }
    if (do_v) {
      const MapFormat f = map_format(send, recv, n_taps, per_head, false, w_dtype);
      if (int st = launch_transpose_maps(wt_v, w.wv, f.batch, f.R, f.C, f.mode, s)) return st;
      wt_v = w.wv;
    }
  }
  const int32_t f_in = n_taps * send->kv_heads * send->head_dim;
  const int32_t f_out = recv->kv_heads * recv->head_dim;

  if (send->dtype == KVX_F32) {
    if (w.tab_send) {
      if (int st = launch_rope_table(w.tab_send, send_tab_rows(send, pos_limit), send->head_dim, send->rope_base, s)) return st;
    }
    if (w.tab_recv) {
      if (int st = launch_rope_table(w.tab_recv, recv_tab_rows_for(recv, pos_limit), recv->head_dim, recv->rope_base, s))
        return st;
    }
    F32Problem p{};
    p.send_layers = send->layers;
    p.send_tokens = send->tokens;
    p.send_heads = send->kv_heads;
    p.send_dim = send->head_dim;
    p.recv_layers = recv->layers;
    p.recv_tokens = recv->tokens;
    p.recv_heads = recv->kv_heads;
    p.recv_dim = recv->head_dim;
    p.n_taps = n_taps;
    p.per_head = per_head ? 1 : 0;
    p.w_f32 = w_dtype == KVX_F32;
    p.taps = taps;
    p.recv_to_send = recv_to_send;
    p.tab_send = w.tab_send;
    p.tab_recv = w.tab_recv;
    F32Role roles[2];
    int n = 0;
    if (do_k)
      roles[n++] = F32Role{static_cast<const float*>(k_send), wt_k, b_k, static_cast<float*>(k_recv),
                           w.tab_send ? 1 : 0, w.tab_recv ? 1 : 0};
    if (do_v) roles[n++] = F32Role{static_cast<const float*>(v_send), wt_v, b_v, static_cast<float*>(v_recv), 0, 0};
    return main_kernel([&] { return launch_f32(p, roles, n, s); });
  }

  // bf16 caches: matrix-core paths, head_dim 128
  if (send->head_dim != 128 || recv->head_dim != 128) return KVX_ERR_UNSUPPORTED;
  if (per_head) {
    const int64_t row_elems = static_cast<int64_t>(send->kv_heads) * 128;
    HeadProblem p{};
    p.send_layers = send->layers;
    p.send_tokens = send->tokens;
    p.recv_layers = recv->layers;
    p.recv_tokens = recv->tokens;
    p.heads = send->kv_heads;
    p.w_f32 = w_dtype == KVX_F32;
    p.taps = taps;
    p.recv_to_send = recv_to_send;
    p.tab_recv = w.tab_recv;
    p.slot = slot;
    p.pool_rows = pool_rows;
    p.recv_pos = recv_pos;
    p.pos_limit = pos_limit;
    HeadRole roles[2];
    int n = 0;
    if (do_k) {
      HeadRole r{};
      if (w.tab_send) {
        // keys rotated back at their sender positions, one fp16 row per run
        if (int st = launch_runs(recv_to_send, recv->tokens, send->tokens, w.runs, w.runs_scratch, s)) return st;
        if (int st = launch_rope_table(w.tab_send, send_tab_rows(send, pos_limit), send->head_dim, send->rope_base, s)) return st;
        uint8_t used[MAX_LAYERS] = {0};
        for (int32_t i = 0; i < recv->layers; ++i) used[taps[i]] = 1;
        if (int st = launch_derotate_rows(static_cast<const uint16_t*>(k_send), send->layers, send->tokens,
                                          send->kv_heads, used, w.runs, w.rows_cap, w.tab_send, send_pos, pos_limit, w.krows, s))
          return st;
        r.x = w.krows;
        r.x_layer_stride = static_cast<int64_t>(w.rows_cap) * row_elems;
        r.x_rows = w.rows_cap;
        r.row_of = w.runs.recv_to_uniq;
        r.x_f16 = 1;
      } else {
        r.x = static_cast<const uint16_t*>(k_send);
        r.x_layer_stride = static_cast<int64_t>(send->tokens) * row_elems;
        r.x_rows = send->tokens;
        r.row_of = recv_to_send;
        r.x_f16 = 0;
      }
      if (w.tab_recv) {
        if (int st = launch_rope_table(w.tab_recv, recv_tab_rows_for(recv, pos_limit), recv->head_dim, recv->rope_base, s))
          return st;
      }
      r.rotate = w.tab_recv ? 1 : 0;
      r.wt = wt_k;
      r.bias = b_k;
      r.out = static_cast<uint16_t*>(k_recv);
      roles[n++] = r;
    }
    if (do_v) {
      HeadRole r{};
      r.x = static_cast<const uint16_t*>(v_send);
      r.x_layer_stride = static_cast<int64_t>(send->tokens) * row_elems;
      r.x_rows = send->tokens;
      r.row_of = recv_to_send;
      r.x_f16 = 0;
      r.rotate = 0;
      r.wt = wt_v;
      r.bias = b_v;
      r.out = static_cast<uint16_t*>(v_recv);
      roles[n++] = r;
    }
    return main_kernel([&] { return launch_perhead(p, roles, n, s); });
  }

  if (f_out % 256 != 0) return KVX_ERR_UNSUPPORTED;
  const int32_t send_row = send->kv_heads * send->head_dim;
  // row offsets inside one sender layer travel as int32
  if (static_cast<int64_t>(send->tokens) * send_row >= (1LL << 31) ||
      static_cast<int64_t>(recv->tokens) * send_row >= (1LL << 31))
    return KVX_ERR_UNSUPPORTED;
  if (int st = launch_runs(recv_to_send, recv->tokens, send->tokens, w.runs, w.runs_scratch, s)) return st;
  const int64_t send_layer_elems = static_cast<int64_t>(send->tokens) * send_row;
  const bool split = w_dtype == KVX_F32;
  FlatRole roles[2];
  int n = 0;
  if (do_k) {
    FlatRole r{};
    if (w.tab_send) {
      if (int st = launch_rope_table(w.tab_send, send_tab_rows(send, pos_limit), send->head_dim, send->rope_base, s)) return st;
      uint8_t used[MAX_LAYERS] = {0};
      for (int32_t i = 0; i < recv->layers * n_taps; ++i) used[taps[i]] = 1;
      if (int st = launch_derotate_rows(static_cast<const uint16_t*>(k_send), send->layers, send->tokens,
                                        send->kv_heads, used, w.runs, w.rows_cap, w.tab_send, send_pos, pos_limit, w.krows, s))
        return st;
      r.a_src = w.krows;
      r.a_layer_stride = static_cast<int64_t>(w.rows_cap) * send_row;
      r.a_compact = 1;
      r.a_f16 = 1;
    } else {
      r.a_src = k_send;
      r.a_layer_stride = send_layer_elems;
      r.a_compact = 0;
      r.a_f16 = 0;
    }
    if (w.tab_recv) {
      if (int st = launch_rope_table(w.tab_recv, recv_tab_rows_for(recv, pos_limit), recv->head_dim, recv->rope_base, s))
        return st;
    }
    // maps in the kernel layout: fp16 for rotated-back keys, bf16 otherwise
    // (fp32 maps as hi|lo halves), or fp8 codes with per-output scales
    r.wt = wt_k;
    if (w_dtype == W_FP8) r.wscale = s_k;
    r.bias = b_k;
    r.out = static_cast<uint16_t*>(k_recv);
    r.rotate = w.tab_recv ? 1 : 0;
    r.knorm = recv->k_norm;
    roles[n++] = r;
  }
  if (do_v) {
    FlatRole r{};
    r.a_src = v_send;
    r.a_layer_stride = send_layer_elems;
    r.a_compact = 0;
    r.a_f16 = 0;
    r.wt = wt_v;
    if (w_dtype == W_FP8) r.wscale = s_v;
    r.bias = b_v;
    r.out = static_cast<uint16_t*>(v_recv);
    r.rotate = 0;
    roles[n++] = r;
  }
  FlatProblem p{};
  p.send_layers = send->layers;
  p.send_tokens = send->tokens;
  p.recv_layers = recv->layers;
  p.recv_tokens = recv->tokens;
  p.k_dim = split ? 2 * f_in : f_in;
  p.f_out = f_out;
  p.n_taps = n_taps;
  p.send_row = send_row;
  p.taps = taps;
  p.tab_recv = w.tab_recv;
  p.runs = w.runs;
  p.knorm_eps = static_cast<float>(recv->k_norm_eps);
  p.slot = slot;
  p.pool_rows = pool_rows;
  p.recv_pos = recv_pos;
  p.pos_limit = pos_limit;
  p.w8 = w_dtype == W_FP8 ? 1 : 0;
  return main_kernel([&] { return launch_flat(p, roles, n, s); });
}

}  // namespace kvx

extern "C" {

int kvx_translate(const kvx_cache_desc* send, const void* k_send, const void* v_send, const kvx_cache_desc* recv,
                  void* k_recv, void* v_recv, const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps,
                  int32_t per_head, int32_t w_dtype, const void* wt_k, const void* wt_v, const float* b_k,
                  const float* b_v, void* workspace, size_t ws_bytes, void* stream) {
  return translate_impl(send, k_send, v_send, recv, k_recv, v_recv, recv_to_send, taps, n_taps, per_head, w_dtype,
                        wt_k, wt_v, b_k, b_v, workspace, ws_bytes, stream, nullptr, nullptr, true);
}

size_t kvx_translate_placed_workspace_size(const kvx_cache_desc* send, const kvx_cache_desc* recv, int32_t n_taps,
                                           int32_t per_head, int32_t pos_limit) {
  if (!desc_ok(send) || !desc_ok(recv) || n_taps < 1 || n_taps > MAX_TAPS || pos_limit < 0) return 0;
  return layout_translate(send, recv, n_taps, per_head, KVX_F32, true, true, pos_limit, true, nullptr).bytes;
}

int kvx_translate_placed(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                         const kvx_cache_desc* recv, void* k_recv, void* v_recv, const int32_t* recv_to_send,
                         const int32_t* taps, int32_t n_taps, int32_t per_head, int32_t w_dtype, const void* wt_k,
                         const void* wt_v, const float* b_k, const float* b_v, void* workspace, size_t ws_bytes,
                         void* stream, const kvx_placement* place) {
  return translate_impl(send, k_send, v_send, recv, k_recv, v_recv, recv_to_send, taps, n_taps, per_head, w_dtype,
                        wt_k, wt_v, b_k, b_v, workspace, ws_bytes, stream, nullptr, place, true);
}

}  // extern "C"

namespace kvx {
// Runs `call(ev)` with three events (before the preparation kernels, before
// and after the main kernel) and reports the two phases in stage_ms.
template <typename F>
static int timed_call(void* stream, float* stage_ms, F&& call) {
  stage_ms[0] = stage_ms[1] = 0.0f;
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  for (auto& e : ev)
    if (hipEventCreate(&e) != hipSuccess) {
      for (auto& f : ev)
        if (f) (void)hipEventDestroy(f);
      return KVX_ERR_HIP;
    }
  int st = call(ev);
  if (st == KVX_OK) {
    // events exist only when work was launched (empty problems return early)
    if (hipEventSynchronize(ev[2]) != hipSuccess ||
        hipEventElapsedTime(&stage_ms[0], ev[0], ev[1]) != hipSuccess ||
        hipEventElapsedTime(&stage_ms[1], ev[1], ev[2]) != hipSuccess) {
      stage_ms[0] = stage_ms[1] = 0.0f;
      if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) st = KVX_ERR_HIP;
    }
  }
  for (auto& e : ev) (void)hipEventDestroy(e);
  return st;
}
}  // namespace kvx

extern "C" {

int kvx_translate_timed(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                        const kvx_cache_desc* recv, void* k_recv, void* v_recv, const int32_t* recv_to_send,
                        const int32_t* taps, int32_t n_taps, int32_t per_head, int32_t w_dtype, const void* wt_k,
                        const void* wt_v, const float* b_k, const float* b_v, void* workspace, size_t ws_bytes,
                        void* stream, float* stage_ms) {
  if (!stage_ms) return KVX_ERR_INVALID;
  return timed_call(stream, stage_ms, [&](hipEvent_t* ev) {
    return translate_impl(send, k_send, v_send, recv, k_recv, v_recv, recv_to_send, taps, n_taps, per_head, w_dtype,
                          wt_k, wt_v, b_k, b_v, workspace, ws_bytes, stream, ev, nullptr, true);
  });
}

int kvx_translate_recorded(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                           const kvx_cache_desc* recv, void* k_recv, void* v_recv, const int32_t* recv_to_send,
                           const int32_t* taps, int32_t n_taps, int32_t per_head, int32_t w_dtype, const void* wt_k,
                           const void* wt_v, const float* b_k, const float* b_v, void* workspace, size_t ws_bytes,
                           void* stream, void* const* events) {
  if (!events || !events[0] || !events[1] || !events[2]) return KVX_ERR_INVALID;
  hipEvent_t ev[3] = {static_cast<hipEvent_t>(events[0]), static_cast<hipEvent_t>(events[1]),
                      static_cast<hipEvent_t>(events[2])};
  return translate_impl(send, k_send, v_send, recv, k_recv, v_recv, recv_to_send, taps, n_taps, per_head, w_dtype,
                        wt_k, wt_v, b_k, b_v, workspace, ws_bytes, stream, ev, nullptr, true);
}

int kvx_translate_prepared(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                           const kvx_cache_desc* recv, void* k_recv, void* v_recv, const int32_t* recv_to_send,
                           const int32_t* taps, int32_t n_taps, int32_t per_head, int32_t w_dtype, const void* pk,
                           const void* pv, const float* b_k, const float* b_v, void* workspace, size_t ws_bytes,
                           void* stream, const kvx_placement* place, void* const* events) {
  if (w_dtype != KVX_F32 && w_dtype != KVX_BF16) return KVX_ERR_INVALID;
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  if (events) {
    if (!events[0] || !events[1] || !events[2]) return KVX_ERR_INVALID;
    for (int i = 0; i < 3; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
  }
  return translate_impl(send, k_send, v_send, recv, k_recv, v_recv, recv_to_send, taps, n_taps, per_head, w_dtype,
                        pk, pv, b_k, b_v, workspace, ws_bytes, stream, events ? ev : nullptr, place, false);
}

int kvx_translate_fp8(const kvx_cache_desc* send, const void* k_send, const void* v_send, const kvx_cache_desc* recv,
                      void* k_recv, void* v_recv, const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps,
                      const uint8_t* wq_k, const uint8_t* wq_v, const float* s_k, const float* s_v, const float* b_k,
                      const float* b_v, void* workspace, size_t ws_bytes, void* stream, float* stage_ms) {
  auto call = [&](hipEvent_t* ev) {
    return translate_impl(send, k_send, v_send, recv, k_recv, v_recv, recv_to_send, taps, n_taps, 0, W_FP8, wq_k,
                          wq_v, b_k, b_v, workspace, ws_bytes, stream, ev, nullptr, false, s_k, s_v);
  };
  if (!stage_ms) return call(nullptr);
  return timed_call(stream, stage_ms, call);
}

int kvx_quantize_fp8(const float* w, int32_t count, int32_t f_in, int32_t f_out, uint8_t* q_out, float* scale_out,
                     void* stream) {
  if (count < 0 || f_in < 1 || f_out < 1) return KVX_ERR_INVALID;
  if (count == 0) return KVX_OK;
  if (count > 65535) return KVX_ERR_UNSUPPORTED;
  if (!w || !q_out || !scale_out) return KVX_ERR_INVALID;
  return launch_quantize_fp8(w, count, f_in, f_out, q_out, scale_out, static_cast<hipStream_t>(stream));
}

int kvx_gather_features(const kvx_cache_desc* send, const void* kv_send, int32_t derotate,
                        const int32_t* recv_to_send, int32_t n_rows, const int32_t* taps_of_layer, int32_t n_taps,
                        void* x_out, void* stream) {
  if (!desc_ok(send) || n_rows < 0 || n_taps < 1 || n_taps > MAX_TAPS || !taps_of_layer) return KVX_ERR_INVALID;
  if (n_rows == 0) return KVX_OK;
  if (!kv_send || !recv_to_send || !x_out) return KVX_ERR_INVALID;
  if (send->tokens == 0) return KVX_ERR_SHAPE;
  if (derotate && !(send->rope_base > 0.0)) return KVX_ERR_INVALID;
  for (int32_t t = 0; t < n_taps; ++t)
    if (taps_of_layer[t] < 0 || taps_of_layer[t] >= send->layers) return KVX_ERR_INVALID;
  const int32_t row = send->kv_heads * send->head_dim;
  if (!derotate && (row % 2) != 0) return KVX_ERR_UNSUPPORTED;
  const int64_t stride = static_cast<int64_t>(send->tokens) * row;
  return launch_gather(kv_send, send->dtype == KVX_F32, send->tokens, row, stride, taps_of_layer, n_taps,
                       recv_to_send, n_rows, derotate ? send->rope_base : 0.0, send->head_dim, x_out,
                       static_cast<hipStream_t>(stream));
}

size_t kvx_fit_ridge_workspace_size(int32_t f_in, int32_t f_out) { return kvx_fit_ridge_batched_workspace_size(1, f_in, f_out); }

static bool fit_size_ok(int32_t count, int32_t f_in, int32_t f_out) {
  return count <= KVX_MAX_PROBLEMS && f_in <= KVX_MAX_FIT_FEATURES && f_out <= KVX_MAX_FIT_FEATURES;
}

size_t kvx_fit_ridge_batched_workspace_size(int32_t count, int32_t f_in, int32_t f_out) {
  if (count < 1 || f_in < 1 || f_out < 1 || !fit_size_ok(count, f_in, f_out)) return 0;
  return fit_ws_bytes(count, f_in, f_out);
}

int kvx_fit_ridge_batched(int32_t count, const void* const* x, int64_t ldx, const void* const* y, int64_t ldy,
                          int32_t in_dtype, int64_t n_rows, int32_t f_in, int32_t f_out, double lambda_abs,
                          double lambda_rel, int32_t fit_intercept, float* const* w_out, float* const* b_out,
                          int32_t* status, void* workspace, size_t ws_bytes, void* stream) {
  if (count < 0 || f_in < 1 || f_out < 1 || n_rows < 0) return KVX_ERR_INVALID;
  if (count == 0) return KVX_OK;
  if (!fit_size_ok(count, f_in, f_out)) return KVX_ERR_UNSUPPORTED;
  if (in_dtype != KVX_F32 && in_dtype != KVX_BF16) return KVX_ERR_INVALID;
  if (!(lambda_abs >= 0.0) || !(lambda_rel >= 0.0)) return KVX_ERR_INVALID;
  if (!x || !y || !w_out || (fit_intercept && !b_out)) return KVX_ERR_INVALID;
  for (int32_t z = 0; z < count; ++z) {
    if (!w_out[z] || (fit_intercept && !b_out[z])) return KVX_ERR_INVALID;
    if (n_rows > 0 && (!x[z] || !y[z])) return KVX_ERR_INVALID;
  }
  if (ldx < f_in || ldy < f_out) return KVX_ERR_SHAPE;
  if (in_dtype == KVX_BF16) {
    // bf16 rows are read in 16-byte pieces
    if ((f_in % 8) || (f_out % 8) || (ldx % 8) || (ldy % 8)) return KVX_ERR_UNSUPPORTED;
    for (int32_t z = 0; z < count; ++z)
      if ((reinterpret_cast<uintptr_t>(x[z]) | reinterpret_cast<uintptr_t>(y[z])) % 16) return KVX_ERR_UNSUPPORTED;
  }
  if (!workspace || ws_bytes < kvx_fit_ridge_batched_workspace_size(count, f_in, f_out)) return KVX_ERR_WORKSPACE;
  return launch_fit(count, x, ldx, y, ldy, in_dtype == KVX_F32, n_rows, f_in, f_out, lambda_abs, lambda_rel,
                    fit_intercept, w_out, b_out, status, workspace, static_cast<hipStream_t>(stream));
}

size_t kvx_fit_recolor_workspace_size(int32_t count, int32_t f_in, int32_t f_out) {
  if (count < 1 || f_in < 1 || f_out < 1 || !fit_size_ok(count, f_in, f_out)) return 0;
  return recolor_ws_bytes(count, f_in, f_out);
}

int kvx_fit_recolor(int32_t count, const void* const* x, int64_t ldx, const void* const* y, int64_t ldy,
                    int32_t in_dtype, int64_t n_rows, int32_t f_in, int32_t f_out, double rho_x, double rho_y,
                    float* const* w_out, float* const* b_out, int32_t* status, int32_t* iters, void* workspace,
                    size_t ws_bytes, void* stream) {
  if (count < 0 || f_in < 1 || f_out < 1 || n_rows < 0) return KVX_ERR_INVALID;
  if (count == 0) return KVX_OK;
  if (!fit_size_ok(count, f_in, f_out)) return KVX_ERR_UNSUPPORTED;
  if (in_dtype != KVX_F32 && in_dtype != KVX_BF16) return KVX_ERR_INVALID;
  if (!(rho_x >= 0.0) || !(rho_y >= 0.0)) return KVX_ERR_INVALID;
  if (!x || !y || !w_out || !b_out) return KVX_ERR_INVALID;
  for (int32_t z = 0; z < count; ++z) {
    if (!w_out[z] || !b_out[z]) return KVX_ERR_INVALID;
    if (n_rows > 0 && (!x[z] || !y[z])) return KVX_ERR_INVALID;
  }
  if (ldx < f_in || ldy < f_out) return KVX_ERR_SHAPE;
  if (f_in < f_out) return KVX_ERR_UNSUPPORTED;
  if (in_dtype == KVX_BF16) {
    if ((f_in % 8) || (f_out % 8) || (ldx % 8) || (ldy % 8)) return KVX_ERR_UNSUPPORTED;
    for (int32_t z = 0; z < count; ++z)
      if ((reinterpret_cast<uintptr_t>(x[z]) | reinterpret_cast<uintptr_t>(y[z])) % 16) return KVX_ERR_UNSUPPORTED;
  }
  if (!workspace || ws_bytes < kvx_fit_recolor_workspace_size(count, f_in, f_out)) return KVX_ERR_WORKSPACE;
  return launch_recolor(count, x, ldx, y, ldy, in_dtype == KVX_F32, n_rows, f_in, f_out, rho_x, rho_y, w_out, b_out,
                        status, iters, workspace, static_cast<hipStream_t>(stream));
}

// Shape of a fit from the caches; false when the descriptors or taps do not
// describe one (sizes as documented in kvx.h).
static bool fitc_shape(const kvx_cache_desc* send, const kvx_cache_desc* recv, int32_t n_taps, int32_t n_roles,
                       FitcShape* sh) {
  if (!desc_ok(send) || !desc_ok(recv) || n_taps < 1 || n_taps > MAX_TAPS) return false;
  sh->send_layers = send->layers;
  sh->n_send = send->tokens;
  sh->row = send->kv_heads * send->head_dim;
  sh->recv_layers = recv->layers;
  sh->n_recv = recv->tokens;
  sh->f_out = recv->kv_heads * recv->head_dim;
  sh->n_taps = n_taps;
  sh->f_in = n_taps * sh->row;
  sh->n_roles = n_roles;
  sh->count = n_roles * recv->layers;
  sh->send_rope = send->rope_base;
  sh->recv_rope = recv->rope_base;
  sh->send_hd = send->head_dim;
  sh->recv_hd = recv->head_dim;
  sh->key_role = -1;
  return true;
}

// Arguments shared by the two fits from the caches: KVX_OK when they describe
// one (the caller checks its own outputs), else the status to return.
static int fitc_check(const kvx_cache_desc* send, const void* k_send, const void* v_send, const kvx_cache_desc* recv,
                      const void* k_recv, const void* v_recv, const int32_t* recv_to_send, const int32_t* taps,
                      int32_t n_taps, bool do_k, bool do_v, FitcShape* sh) {
  const int32_t n_roles = (do_k ? 1 : 0) + (do_v ? 1 : 0);
  if (n_roles == 0 || !fitc_shape(send, recv, n_taps, n_roles, sh)) return KVX_ERR_INVALID;
  if ((do_k && (!k_send || !k_recv)) || (do_v && (!v_send || !v_recv))) return KVX_ERR_INVALID;
  if (!taps || (recv->tokens > 0 && !recv_to_send)) return KVX_ERR_INVALID;
  for (int32_t i = 0; i < recv->layers * n_taps; ++i)
    if (taps[i] < 0 || taps[i] >= send->layers) return KVX_ERR_INVALID;
  if (send->dtype != KVX_BF16 || recv->dtype != KVX_BF16) return KVX_ERR_UNSUPPORTED;
  // rotated keys are turned back in pieces of 8 pairs (c .. c+7, c+d/2 .. c+d/2+7)
  if ((send->rope_base > 0.0 && send->head_dim % 16) || (recv->rope_base > 0.0 && recv->head_dim % 16))
    return KVX_ERR_UNSUPPORTED;
  sh->key_role = do_k ? 0 : -1;
  if ((sh->row % 256) != 0 || (sh->f_out % 8) != 0) return KVX_ERR_UNSUPPORTED;
  // rows are read in 16-byte pieces
  for (const void* p : {k_send, v_send, k_recv, v_recv})
    if (reinterpret_cast<uintptr_t>(p) % 16) return KVX_ERR_UNSUPPORTED;
  if (sh->f_in > KVX_MAX_FIT_FEATURES || sh->f_out > KVX_MAX_FIT_FEATURES) return KVX_ERR_UNSUPPORTED;
  if (sh->n_recv < 1 || sh->n_send < 1) return KVX_ERR_SHAPE;
  // the Gram's per-layer operands are addressed with 32-bit byte offsets
  const int64_t widest = sh->row > sh->f_out ? sh->row : sh->f_out;
  if (fitc_max_rows(*sh) * widest * 2 >= (1LL << 31)) return KVX_ERR_UNSUPPORTED;
  return KVX_OK;
}

size_t kvx_fit_ridge_caches_workspace_size(const kvx_cache_desc* send, const kvx_cache_desc* recv, int32_t n_taps) {
  FitcShape sh{};
  if (!fitc_shape(send, recv, n_taps, 2, &sh) || sh.n_recv < 1) return 0;
  if (sh.f_in > KVX_MAX_FIT_FEATURES || sh.f_out > KVX_MAX_FIT_FEATURES) return 0;
  return fitc_ws_bytes(sh);
}

int kvx_fit_ridge_caches(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                         const kvx_cache_desc* recv, const void* k_recv, const void* v_recv,
                         const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps, double lambda_abs,
                         double lambda_rel, float* w_k, float* w_v, int32_t* status, void* workspace,
                         size_t ws_bytes, void* stream) {
  FitcShape sh{};
  if (int st = fitc_check(send, k_send, v_send, recv, k_recv, v_recv, recv_to_send, taps, n_taps, w_k != nullptr,
                          w_v != nullptr, &sh))
    return st;
  if (!(lambda_abs >= 0.0) || !(lambda_rel >= 0.0)) return KVX_ERR_INVALID;
  if (!workspace || ws_bytes < fitc_ws_bytes(sh)) return KVX_ERR_WORKSPACE;
  const void* sends[2];
  const void* recvs[2];
  float* outs[2];
  int32_t r = 0;
  if (w_k) {
    sends[r] = k_send;
    recvs[r] = k_recv;
    outs[r++] = w_k;
  }
  if (w_v) {
    sends[r] = v_send;
    recvs[r] = v_recv;
    outs[r++] = w_v;
  }
  int32_t st_roles[2 * MAX_LAYERS];
  const int st = launch_fit_caches(sh, sends, recvs, recv_to_send, taps, lambda_abs, lambda_rel, outs, st_roles,
                                   workspace, static_cast<hipStream_t>(stream));
  if (status && (st == KVX_OK || st == KVX_ERR_NOT_SPD)) {
    // [2][L_R]: a skipped role's entries are KVX_OK
    int32_t z = 0;
    for (int32_t role = 0; role < 2; ++role) {
      const bool present = role == 0 ? w_k != nullptr : w_v != nullptr;
      for (int32_t l = 0; l < recv->layers; ++l) status[role * recv->layers + l] = present ? st_roles[z++] : KVX_OK;
    }
  }
  return st;
}

size_t kvx_fit_recolor_caches_workspace_size(const kvx_cache_desc* send, const kvx_cache_desc* recv,
                                             int32_t n_taps) {
  FitcShape sh{};
  if (!fitc_shape(send, recv, n_taps, 2, &sh) || sh.n_recv < 1) return 0;
  if (sh.f_in > KVX_MAX_FIT_FEATURES || sh.f_out > KVX_MAX_FIT_FEATURES) return 0;
  return recolor_caches_ws_bytes(sh);
}

int kvx_fit_recolor_caches(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                           const kvx_cache_desc* recv, const void* k_recv, const void* v_recv,
                           const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps, double rho_x,
                           double rho_y, float* w_k, float* w_v, float* b_k, float* b_v, int32_t* status,
                           int32_t* iters, void* workspace, size_t ws_bytes, void* stream) {
  FitcShape sh{};
  if (int st = fitc_check(send, k_send, v_send, recv, k_recv, v_recv, recv_to_send, taps, n_taps, w_k != nullptr,
                          w_v != nullptr, &sh))
    return st;
  if (!(rho_x >= 0.0) || !(rho_y >= 0.0)) return KVX_ERR_INVALID;
  if ((w_k && !b_k) || (w_v && !b_v)) return KVX_ERR_INVALID;  // the bias is always written
  if (sh.f_in < sh.f_out) return KVX_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < recolor_caches_ws_bytes(sh)) return KVX_ERR_WORKSPACE;
  const void* sends[2];
  const void* recvs[2];
  float* ws_[2];
  float* bs_[2];
  int32_t r = 0;
  if (w_k) {
    sends[r] = k_send;
    recvs[r] = k_recv;
    ws_[r] = w_k;
    bs_[r++] = b_k;
  }
  if (w_v) {
    sends[r] = v_send;
    recvs[r] = v_recv;
    ws_[r] = w_v;
    bs_[r++] = b_v;
  }
  int32_t st_roles[2 * MAX_LAYERS];
  const int st = launch_recolor_caches(sh, sends, recvs, recv_to_send, taps, rho_x, rho_y, ws_, bs_, st_roles, iters,
                                       workspace, static_cast<hipStream_t>(stream));
  if (status && (st == KVX_OK || st == KVX_ERR_NOT_SPD || st == KVX_ERR_NOT_CONVERGED)) {
    int32_t z = 0;
    for (int32_t role = 0; role < 2; ++role) {
      const bool present = role == 0 ? w_k != nullptr : w_v != nullptr;
      for (int32_t l = 0; l < recv->layers; ++l) status[role * recv->layers + l] = present ? st_roles[z++] : KVX_OK;
    }
  }
  return st;
}

int kvx_fit_ridge(const void* x, int64_t ldx, const void* y, int64_t ldy, int32_t in_dtype, int64_t n_rows,
                  int32_t f_in, int32_t f_out, double lambda_abs, double lambda_rel, int32_t fit_intercept,
                  float* w_out, float* b_out, void* workspace, size_t ws_bytes, void* stream) {
  return kvx_fit_ridge_batched(1, &x, ldx, &y, ldy, in_dtype, n_rows, f_in, f_out, lambda_abs, lambda_rel,
                               fit_intercept, &w_out, &b_out, nullptr, workspace, ws_bytes, stream);
}

int kvx_probe_hbm(int32_t mode, void* a, void* b, int64_t bytes, int32_t iters, float* ms_per_launch, void* stream) {
  if (mode < 0 || mode > 2 || bytes < 16 || (bytes % 16) != 0 || iters < 1 || !a || !ms_per_launch)
    return KVX_ERR_INVALID;
  if (mode != 2 && !b) return KVX_ERR_INVALID;
  return run_probe_hbm(mode, a, b, bytes, iters, ms_per_launch, static_cast<hipStream_t>(stream));
}

int kvx_probe_mfma(float* out, int32_t reps, int32_t iters, float* ms_per_launch, double* flops_per_launch,
                   void* stream) {
  if (!out || reps < 1 || iters < 1 || !ms_per_launch || !flops_per_launch) return KVX_ERR_INVALID;
  return run_probe_mfma(out, reps, iters, ms_per_launch, flops_per_launch, static_cast<hipStream_t>(stream));
}

int32_t kvx_probe_scratch_words(void) {
  const int a = probe_mfma_out_floats(), b = probe_read_sink_words();
  return a > b ? a : b;
}

int kvx_fold_lowrank(const float* w, const float* a, const float* b, int32_t count, int32_t f_in, int32_t f_out,
                     int32_t rank, void* w_out, int32_t out_dtype, void* stream) {
  if (count < 0 || f_in < 1 || f_out < 1 || rank < 0) return KVX_ERR_INVALID;
  if (out_dtype != KVX_F32 && out_dtype != KVX_BF16) return KVX_ERR_INVALID;
  if (count == 0) return KVX_OK;
  if (!w || !w_out || (rank > 0 && (!a || !b))) return KVX_ERR_INVALID;
  return launch_fold(w, a, b, count, f_in, f_out, rank, w_out, out_dtype == KVX_BF16,
                     static_cast<hipStream_t>(stream));
}

}  // extern "C"
