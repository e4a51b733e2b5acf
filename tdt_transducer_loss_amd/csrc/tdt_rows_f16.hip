// Row kernels of the TDT loss instantiated for f16 logits.
#include "tdt_kernels.h"
#include "tdt_rows.h"

namespace tdt {
hipError_t launch_rows_f16(const Params& p, bool aligned, hipStream_t st, int which) {
  return launch_rows_t<F16>(p, aligned, st, which);
}
}  // namespace tdt
