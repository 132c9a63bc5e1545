// Launchers of the moment-matched (Recolor) fit, shared between the fit and
// the C-ABI translation units.
#pragma once

#include "kvx_internal.hpp"

namespace kvx {

size_t recolor_ws_bytes(int32_t count, int32_t f_in, int32_t f_out);
// `count` problems of one shape (f_in >= f_out); x, y, w_out, b_out are host
// arrays of device pointers; status (host, may be null) receives each
// problem's status; iters (host, may be null) receives the number of polar
// iterations run.
int launch_recolor(int32_t count, const void* const* x, int64_t ldx, const void* const* y, int64_t ldy,
                   int32_t in_f32, int64_t n_rows, int32_t f_in, int32_t f_out, double rho_x, double rho_y,
                   float* const* w_out, float* const* b_out, int32_t* status, int32_t* iters, void* ws,
                   hipStream_t s);

// Ridge fits of every receiver layer of n_roles roles from the calibration
// caches (kvx_fit_ridge_caches): shapes, host arrays of the roles' cache
// pointers and outputs; problems role by role, receiver layer within.
struct FitcShape {
  int32_t send_layers, n_send, row;        // sender: layers, tokens, H_S d_S (a multiple of 256)
  int32_t recv_layers, n_recv, f_out;      // receiver: layers, tokens, H_R d_R
  int32_t n_taps, f_in, n_roles, count;    // f_in = n_taps row, count = n_roles recv_layers
  // keys stored rotated (base > 0): the sender's rotated back at the sender
  // position, the receiver's (the targets) at the receiver position; head
  // dims for the pairs (c, c + d/2); key_role = index of the key role among
  // the roles fitted, or -1
  double send_rope, recv_rope;
  int32_t send_hd, recv_hd, key_role;
};
size_t fitc_ws_bytes(const FitcShape& sh);
// the most rows a per-layer operand of the Gram can have (for the 32-bit
// offset limit of its loads)
int64_t fitc_max_rows(const FitcShape& sh);
int launch_fit_caches(const FitcShape& sh, const void* const* send_role, const void* const* recv_role,
                      const int32_t* map, const int32_t* taps_host, double lam_abs, double lam_rel,
                      float* const* w_role, int32_t* status, void* ws, hipStream_t s);
// Recolor fits of every receiver layer of n_roles roles from the calibration
// caches (kvx_fit_recolor_caches); status and iters as for launch_recolor.
size_t recolor_caches_ws_bytes(const FitcShape& sh);
int launch_recolor_caches(const FitcShape& sh, const void* const* send_role, const void* const* recv_role,
                          const int32_t* map, const int32_t* taps_host, double rho_x, double rho_y,
                          float* const* w_role, float* const* b_role, int32_t* status, int32_t* iters, void* ws,
                          hipStream_t s);

}  // namespace kvx
