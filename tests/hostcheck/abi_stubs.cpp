// Stand-ins for the HIP side of the library, for a host-only build of the
// C-ABI layer (fa_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every launcher returns success without
// touching a device, so the sanitized library exercises exactly the
// argument validation and dispatch of fa_api.cpp.  The tile grids repeat
// the kernels' values (the ABI tests compare them with the real library's).
#include "../../exact_io_aware_amd/csrc/fa_internal.h"

namespace fa {

hipError_t launch_fwd_bf16(const FwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_splitkv_bf16(const SplitKvArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_fwd_f32(const FwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_preprocess(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_dkdv(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_dq(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_dq_stats(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_preprocess_f32(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_dkdv_f32(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_dq_f32(const BwdArgs&, hipStream_t) { return hipSuccess; }

void fwd_bf16_tile_grid(int d, bool sparse, int* rows, int* cols) {
  *rows = (d == 128 && !sparse) ? 256 : 128;
  *cols = (d == 128) ? 64 : 128;
}
void bwd_dkdv_tile_grid(int d, bool sparse, int* rows, int* cols) {
  if (d == 128 && !sparse) {
    *rows = 32;
    *cols = 256;
    return;
  }
  *rows = (d == 128) ? 64 : 128;
  *cols = 128;
}
void bwd_dq_tile_grid(int d, bool sparse, int* rows, int* cols) {
  *rows = (d == 128 && !sparse) ? 256 : 128;
  *cols = (d == 128) ? 64 : 128;
}

size_t noalloc_scratch_bytes() { return (size_t)8 << 20; }
hipError_t noalloc_scratch(void** out) {
  *out = reinterpret_cast<void*>((uintptr_t)4096);  // never dereferenced
  return hipSuccess;
}

}  // namespace fa
