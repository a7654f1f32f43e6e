// MFMA (bf16, d = 128) DropKV path for gfx950.
#include "dropkv_common.h"

namespace dropkv {

bool mfma_supported(int dtype, int d) { return false && dtype == 0 && d == 128; }

int mfma_chunks(const Shape& s) { (void)s; return 1; }

hipError_t launch_mfma_path(const void*, const void*, const void*, const Shape&, const Workspace&,
                            hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace dropkv
