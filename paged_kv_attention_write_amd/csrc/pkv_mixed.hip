// Mixed chunked-prefill + decode step (prefill tiles on the matrix cores).
#include "pkv_attention.h"

namespace pkv {

int launch_mixed(const AttnArgs&, int, int, int, int, int, void*) { return PKV_ERR_UNSUPPORTED; }

}  // namespace pkv
