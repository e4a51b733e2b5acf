// Row kernels of the TDT loss instantiated for bf16 logits.
#include "tdt_kernels.h"
#include "tdt_rows.h"

namespace tdt {
hipError_t launch_rows_bf16(const Params& p, bool aligned, hipStream_t st, int which) {
  return launch_rows_t<BF16>(p, aligned, st, which);
}
}  // namespace tdt
