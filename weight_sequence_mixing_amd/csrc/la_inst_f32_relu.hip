// Instantiations: fp32 inputs (fp32 matrix-core path), ReLU feature map.
#include "la_decode.h"
#include "la_forward.h"

namespace la {
#define LA_ENTRY(T, TCODE, PHI, DK, F, DV) \
    {TCODE, PHI, DK, F, DV, chunk_len<T, PHI>(F), &fwd_launch<T, PHI, DK, F, DV>, &dec_launch<T, PHI, DK, F, DV>}

KernelEntry kEntriesF32Relu[] = {
    LA_ENTRY(float, LA_F32, LA_PHI_RELU, 64, 64, 64),
    LA_ENTRY(float, LA_F32, LA_PHI_RELU, 64, 64, 128),
    LA_ENTRY(float, LA_F32, LA_PHI_RELU, 128, 128, 64),
    LA_ENTRY(float, LA_F32, LA_PHI_RELU, 128, 128, 128),
};
int kNumEntriesF32Relu = sizeof(kEntriesF32Relu) / sizeof(kEntriesF32Relu[0]);
}  // namespace la
