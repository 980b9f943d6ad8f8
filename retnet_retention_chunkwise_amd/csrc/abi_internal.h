// Pieces of the C-ABI layer (api.cpp) shared with entry points defined in
// other sources: the chunkwise forward split into validation and launch, and
// the thread-local error text.
#pragma once

#include <stddef.h>

#include "libretention.h"

namespace ret {

struct ChunkwiseFwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;  // host, H floats
  const float* state_in;
  float* state_out;
  void* y;
  int B, H, T, dk, dv, C, dt;
};

// Every argument check of retention_chunkwise_fwd; the workspace (pointer,
// size, alignment, overlaps) only when check_ws.  Makes no HIP call; sets the
// error text (naming the entry point fn) on failure.
ret_status chunkwise_fwd_check(const ChunkwiseFwdArgs& a, const void* workspace, size_t workspace_bytes,
                               bool check_ws, const char* fn);

// Kernel choice and launch of a checked call; workspace holds
// retention_chunkwise_workspace_bytes() bytes when that is non-zero.
ret_status chunkwise_fwd_run(const ChunkwiseFwdArgs& a, void* workspace, void* stream);

// Replaces the thread's error text (what retention_last_error returns).
void set_last_error(const char* text);

}  // namespace ret
