// fp8 (e4m3fn) sparse attention: not built yet; the entry point reports it.
#include "fp_launch.h"

hipError_t launch_attn_fp8(const AttnArgs&, const SeqTable&, int, int, hipStream_t) {
    return hipErrorNotSupported;
}
