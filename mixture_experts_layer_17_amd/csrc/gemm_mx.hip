// MXFP8 grouped expert-FFN GEMMs (MX-scaled FP8 MFMA on gfx950).
#include "mx_common.hpp"

namespace moe {

size_t mx_ffn_scratch_bytes(int64_t, int, int, int, int) { return 0; }
int mx_ffn_fwd(const FfnArgs&, int64_t, char*, hipStream_t) { return MOE_EUNSUPPORTED; }
int mx_ffn_bwd(const FfnArgs&, int64_t, const int32_t*, char*, hipStream_t) { return MOE_EUNSUPPORTED; }

}  // namespace moe
