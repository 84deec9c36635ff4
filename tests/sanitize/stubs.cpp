// Device launchers replaced for the host-only sanitizer build: host-only handles never
// launch, so these only satisfy the linker (and report "no device" if ever reached).
#include "plan.h"

namespace sc {
int occupancy(const Plan&, int* cus, int* per_cu) {
  *cus = 256;
  *per_cu = 1;
  return 0;
}
int launch_sparse(const Plan&, const KArgs&, void*, int) { return 100; }
int launch_escoin(const EscoinArgs&, const float*, float*, float*, const uint32_t*, const int32_t*, void*) {
  return 100;
}
int launch_dense(DenseArgs, const float*, const float*, float*, int, void*) { return 100; }
int scratch_address(void** ptr) {
  *ptr = nullptr;
  return 100;
}
}  // namespace sc
