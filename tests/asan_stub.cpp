// Host-only stand-ins for the device half of the library, linked with the
// phase-1 planner into an AddressSanitizer build that the CPU tests load
// (tests/test_host_asan.py).  Every entry point that would launch device work
// returns FA_ERR_RUNTIME instead.
#include <stdint.h>

#include "fa_fwd.h"
#include "fa_merge.h"
#include "fa_plan.h"

namespace fa {
int merge_launch(const MergeParams&, int32_t, void*) { return 1; }
}  // namespace fa

extern "C" fa_status fa_fwd(void*, uint64_t, const fa_plan*, void*) {
  fa_set_error("host-only build: no device");
  return FA_ERR_RUNTIME;
}

extern "C" fa_status fa_fwd_noalloc(const fa_plan*, void*) {
  fa_set_error("host-only build: no device");
  return FA_ERR_RUNTIME;
}

extern "C" fa_status fa_clock_probe(uint32_t, unsigned long long*, void*) {
  fa_set_error("host-only build: no device");
  return FA_ERR_RUNTIME;
}
