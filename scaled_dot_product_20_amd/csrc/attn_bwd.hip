// attn_bwd.hip - the backward's dtype dispatch (each dtype's kernels are
// built in their own file from attn_bwd_kernels.hpp) and the zero rows of a
// sequence's room past its length.
#include "attn_launch.hpp"

namespace sdpa {

template <class Ex>
static hipError_t launch_bwd_any(int dtype, int head_dim, const BwdArgs& a, int stages, const Ex& ex) {
  hipError_t err;
  switch (dtype) {
    case 0: err = launch_bwd_f32(head_dim, a, stages, ex); break;
    case 1: err = launch_bwd_f16(head_dim, a, stages, ex); break;
    case 2: err = launch_bwd_bf16(head_dim, a, stages, ex); break;
    default: return hipErrorNotSupported;
  }
  // Rows of a sequence's room past its length: dQ, and dK / dV, are zero.
  const int esz = dtype == 0 ? 4 : 2, rb = head_dim * esz;
  if (err == hipSuccess && (stages & kStageDq)) err = launch_pad_rows(a.p, a.dq, Operand{}, nullptr, 0, rb, esz, ex);
  if (err == hipSuccess && (stages & kStageDkDv)) err = launch_pad_rows(a.p, a.dk, a.dv, nullptr, 1, rb, esz, ex);
  return err;
}

hipError_t launch_bwd(int dtype, int head_dim, const BwdArgs& a, int stages, const Enqueue& ex) {
  return launch_bwd_any(dtype, head_dim, a, stages, ex);
}
hipError_t launch_bwd(int dtype, int head_dim, const BwdArgs& a, int stages, const Record& ex) {
  return launch_bwd_any(dtype, head_dim, a, stages, ex);
}

}  // namespace sdpa
