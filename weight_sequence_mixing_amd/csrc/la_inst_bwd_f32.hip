// Instantiations of the backward sweeps: f32 inputs, elementwise feature maps.
#include "la_backward.h"

namespace la {
#define LA_BWD_ENTRY(PHI, DK, DV) {LA_F32, PHI, DK, DK, DV, 32, &bwd_launch<float, PHI, DK, DK, DV>, bwd_dlam_fits<float, DK, DK, DV>()}

BwdEntry kBwdEntriesF32[] = {
    LA_BWD_ENTRY(LA_PHI_ELU1, 64, 64),
    LA_BWD_ENTRY(LA_PHI_ELU1, 64, 128),
    LA_BWD_ENTRY(LA_PHI_ELU1, 128, 64),
    LA_BWD_ENTRY(LA_PHI_ELU1, 128, 128),
    LA_BWD_ENTRY(LA_PHI_RELU, 64, 64),
    LA_BWD_ENTRY(LA_PHI_RELU, 64, 128),
    LA_BWD_ENTRY(LA_PHI_RELU, 128, 64),
    LA_BWD_ENTRY(LA_PHI_RELU, 128, 128),
};
int kNumBwdEntriesF32 = sizeof(kBwdEntriesF32) / sizeof(kBwdEntriesF32[0]);
}  // namespace la
