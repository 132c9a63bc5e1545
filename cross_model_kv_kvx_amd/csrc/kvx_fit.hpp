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

}  // namespace kvx
