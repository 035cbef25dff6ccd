// Backward kernels (placeholder until the backward path lands).
#include "nsa_common.hpp"
#include "nsa_kernels.hpp"
#include "../../include/nsa.h"

namespace nsa {
size_t bwd_ws_bytes(const Dims& dm) { (void)dm; return 0; }
int bwd_stage_count() { return 1; }
hipError_t launch_bwd(const Dims& dm, const nsa_bwd_args* a, void* ws, hipStream_t s, void* const* events) {
  (void)dm; (void)a; (void)ws; (void)s; (void)events;
  return hipErrorNotSupported;
}
}  // namespace nsa
