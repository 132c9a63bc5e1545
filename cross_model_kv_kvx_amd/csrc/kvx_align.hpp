// Launchers of the token alignment that the C-ABI translation unit uses
// beyond those of kvx_internal.hpp.
#pragma once

#include "kvx_internal.hpp"

namespace kvx {

// One sequence without synchronisation: invalid (device int32) receives 1
// when an offset array is not positive and strictly increasing, else 0.
int launch_align_async(const int32_t* send_end, int32_t n_send, const int32_t* recv_end, int32_t n_recv,
                       int32_t* out, int32_t* invalid, void* ws, hipStream_t s);

// The same without a workspace: the scan's scratch is a static device array
// sized for NOALLOC_MAX_RECV receiver tokens (larger n_recv:
// KVX_ERR_WORKSPACE); allocates nothing.
constexpr int32_t NOALLOC_MAX_RECV = 1 << 24;
int launch_align_noalloc(const int32_t* send_end, int32_t n_send, const int32_t* recv_end, int32_t n_recv,
                         int32_t* out, int32_t* invalid, hipStream_t s);

}  // namespace kvx
