// attn_bwd_f32.hip - the fp32 instantiations of the backward kernels and
// their launch rules (attn_bwd_kernels.hpp).
#include "attn_bwd_kernels.hpp"

namespace sdpa {

hipError_t launch_bwd_f32(int head_dim, const BwdArgs& a, int stages, const Enqueue& ex) {
  return launch_bwd_d<MmaF32>(head_dim, a, stages, ex);
}
hipError_t launch_bwd_f32(int head_dim, const BwdArgs& a, int stages, const Record& ex) {
  return launch_bwd_d<MmaF32>(head_dim, a, stages, ex);
}

}  // namespace sdpa
