// Host-only stand-ins for the HIP side of libvdn_local_attn, used to build the
// C-ABI front end (api.cpp) and the scheduler (schedule.cpp) with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every launcher reports
// that no device is present; the tests that load the sanitizer build only reach them
// through calls whose validation passes, which the CPU tests never make.
#include <hip/hip_runtime.h>

#include "../../block_sparse_attention_31_amd/csrc/fwd_params.hpp"
#include "../../block_sparse_attention_31_amd/csrc/linear_params.hpp"

extern "C" const char* hipGetErrorString(hipError_t) { return "no HIP device in the host-only build"; }

namespace vdn {
int kernel_tile_m(int, int) { return 256; }
int bwd_dq_tile_m() { return 256; }
int bwd_dkv_tile_n() { return 256; }
int launch_fwd(const FwdParams&, int, int, void*) { return int(hipErrorNoDevice); }
int launch_fwd_fp8(const FwdParams&, int, void*) { return int(hipErrorNoDevice); }
int launch_bwd(const BwdDqParams&, const BwdKvParams&, int, void*) { return int(hipErrorNoDevice); }
int bwd_scratch(float**) { return int(hipErrorNoDevice); }
int launch_linear(const LinParams&, int, void*) { return int(hipErrorNoDevice); }
int launch_fuse(const FuseParams&, void*) { return int(hipErrorNoDevice); }
}  // namespace vdn
