// Host interface of the full-BPTT gradient of the replay (fp32 arithmetic).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <string>
#include <utility>

#include "rlt.h"

namespace rlt {

// Bytes of device workspace the gradient needs for B sequences of T positions (checkpoint:
// keep block inputs, keys and values only, and recompute the rest before each backward).
size_t grad_workspace_bytes(const rlt_config& c, int B, int T, bool checkpoint);

// Runs the saved-activation forward, the loss gradient, the reverse-time decoder
// scan and the encoder backward on `stream`. W: every manifest weight (fp32, device);
// G: every manifest gradient buffer (fp32, device) with its element count, zeroed here first. Decoder
// weights of a shared configuration resolve to the encoder layer's entries in both.
// Shapes and names are validated by the caller. Returns the first HIP error.
hipError_t replay_grad(const rlt_config& c, const std::map<std::string, const float*>& W,
                       const std::map<std::string, std::pair<float*, int64_t>>& G, const int32_t* tokens, int B, int T,
                       const float* dlogprob, float* logprob, void* workspace, bool checkpoint, hipStream_t stream);

}  // namespace rlt
