// Instantiations of the backward sweeps: bf16 inputs, elementwise feature maps.
#include "la_backward.h"

namespace la {
#define LA_BWD_ENTRY(PHI, DK, DV) {LA_BF16, PHI, DK, DK, DV, 32, &bwd_launch<bf16, PHI, DK, DK, DV>, bwd_dlam_fits<bf16, DK, DK, DV>()}

BwdEntry kBwdEntriesBf16[] = {
    LA_BWD_ENTRY(LA_PHI_ELU1, 64, 64),
    LA_BWD_ENTRY(LA_PHI_ELU1, 64, 128),
    LA_BWD_ENTRY(LA_PHI_ELU1, 128, 64),
    LA_BWD_ENTRY(LA_PHI_ELU1, 128, 128),
    LA_BWD_ENTRY(LA_PHI_RELU, 64, 64),
    LA_BWD_ENTRY(LA_PHI_RELU, 64, 128),
    LA_BWD_ENTRY(LA_PHI_RELU, 128, 64),
    LA_BWD_ENTRY(LA_PHI_RELU, 128, 128),
};
int kNumBwdEntriesBf16 = sizeof(kBwdEntriesBf16) / sizeof(kBwdEntriesBf16[0]);
}  // namespace la
