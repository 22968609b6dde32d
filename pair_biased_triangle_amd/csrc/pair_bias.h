// Attention with pair bias on one line (I == 1), bf16, D == 32: the single-pass kernel
// that reads the raw bias once (kernel_pair_bias.hip).
#pragma once

#include "launch.h"

namespace tri_attn {

// True when the single-pass kernel takes the call: one line, starting orientation, the
// whole key range, no state output, bf16 with D == 32, N even (the raw bias rows are
// then 4-byte aligned for the row copies) and bias 16-byte aligned.
bool pair_bias_direct_applies(const Problem& p);
// Workspace of the single-pass kernel: the partial states of its key ranges (0 when one range).
size_t pair_bias_direct_workspace_bytes(const Problem& p);
hipError_t launch_pair_bias_direct(const Problem& p, void* workspace, hipStream_t stream);

}  // namespace tri_attn
