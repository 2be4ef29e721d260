// Host-only stand-ins for the device launchers of liblard.so, for a sanitizer build of the
// C-ABI layer (lard_api.cpp) on a machine without a GPU: every launch reports a failure,
// which the entry points map to LARD_ERR_HIP.  Test infrastructure only.
#include "probe_internal.h"
#include "relkl_internal.h"

namespace lard {

int launch_fwd(const FwdLaunch&, bool, int, bool, const LossOut&, void*, bool) { return 1; }
int launch_bwd(const BwdLaunch&, bool, int, bool, bool, void*, int) { return 1; }
int launch_splitk_reduce(const ReduceLaunch&, bool, void*) { return 1; }
int launch_rope_prep(const PrepLaunch&, bool, int, void*, bool) { return 1; }
int launch_probe_mfma(bool, int, int, float*, void*) { return 1; }
int scratch_address(void** out) {
  *out = nullptr;
  return 1;
}

}  // namespace lard
