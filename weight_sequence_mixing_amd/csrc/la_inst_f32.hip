// Instantiations: fp32 inputs (fp32 matrix-core path), both feature maps.
#include "la_decode.h"
#include "la_forward.h"

namespace la {
#define LA_ENTRY(T, TCODE, PHI, DK, F, DV) \
    {TCODE, PHI, DK, F, DV, chunk_len<T, PHI>(F), &fwd_launch<T, PHI, DK, F, DV>, &dec_launch<T, PHI, DK, F, DV>}

KernelEntry kEntriesF32[] = {
    LA_ENTRY(float, LA_F32, LA_PHI_ELU1, 64, 64, 64),
    LA_ENTRY(float, LA_F32, LA_PHI_ELU1, 64, 64, 128),
    LA_ENTRY(float, LA_F32, LA_PHI_ELU1, 128, 128, 64),
    LA_ENTRY(float, LA_F32, LA_PHI_ELU1, 128, 128, 128),
    LA_ENTRY(float, LA_F32, LA_PHI_TRIG_RF, 64, 64, 64),
    LA_ENTRY(float, LA_F32, LA_PHI_TRIG_RF, 64, 64, 128),
    LA_ENTRY(float, LA_F32, LA_PHI_TRIG_RF, 64, 128, 64),
    LA_ENTRY(float, LA_F32, LA_PHI_TRIG_RF, 64, 128, 128),
    LA_ENTRY(float, LA_F32, LA_PHI_TRIG_RF, 128, 64, 64),
    LA_ENTRY(float, LA_F32, LA_PHI_TRIG_RF, 128, 64, 128),
    LA_ENTRY(float, LA_F32, LA_PHI_TRIG_RF, 128, 128, 64),
    LA_ENTRY(float, LA_F32, LA_PHI_TRIG_RF, 128, 128, 128),
};
int kNumEntriesF32 = sizeof(kEntriesF32) / sizeof(kEntriesF32[0]);
}  // namespace la
