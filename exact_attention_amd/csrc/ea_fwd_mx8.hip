// MX fp8 forward: placeholder until the scaled-MFMA kernel lands.
#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

hipError_t launch_fwd_mx8(const Mx8Args& a, bool causal, hipStream_t s) {
  (void)a;
  (void)causal;
  (void)s;
  return hipErrorNotSupported;
}

}  // namespace ea
