// Window scoring kernel for f32 states and head_dim 128 (one translation
// unit per instantiation so that the library builds in parallel).

#include "kara_score_kernel.hpp"

namespace kara {
template hipError_t launch_score_typed<float, 128>(const ScoreArgs& a, hipStream_t stream);
}  // namespace kara
