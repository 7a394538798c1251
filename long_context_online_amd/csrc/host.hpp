// Host-side internals shared by the source files of the C ABI.
//
// Error reporting: every entry point returns a status code; the message of the calling thread's
// last error is kept in a thread-local buffer (read with blasst_last_error()), set on every error
// return and cleared on success.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "../../include/blasst.h"

namespace blasst {

// Formats the message of the calling thread's last error and returns st.
blasst_status fail(blasst_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the calling thread's last error and returns BLASST_OK.
blasst_status ok();

// Decode, in two halves: the argument checks (no HIP call; *ws_bytes receives the scratch bytes the
// launch needs, 0 when num_splits == 1 or stats_only), then the launches with the per-split
// partials at `ws` (at least *ws_bytes bytes, 256-byte aligned; ignored when *ws_bytes is 0).
blasst_status decode_validate(const blasst_decode_params *p, size_t *ws_bytes);
blasst_status decode_launch(const blasst_decode_params *p, void *ws, hipStream_t st);

}  // namespace blasst
