// Instantiations: bf16 inputs, trigonometric random features (F = 2m).
#include "la_decode.h"
#include "la_forward.h"

namespace la {
#define LA_ENTRY(T, TCODE, PHI, DK, F, DV) \
    {TCODE, PHI, DK, F, DV, plan_chunk<T, PHI>(F), &fwd_launch<T, PHI, DK, F, DV>, &dec_launch<T, PHI, DK, F, DV>}

KernelEntry kEntriesBf16Rf[] = {
    LA_ENTRY(bf16, LA_BF16, LA_PHI_TRIG_RF, 64, 64, 64),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_TRIG_RF, 64, 64, 128),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_TRIG_RF, 64, 128, 64),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_TRIG_RF, 64, 128, 128),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_TRIG_RF, 64, 256, 64),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_TRIG_RF, 64, 256, 128),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_TRIG_RF, 128, 64, 64),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_TRIG_RF, 128, 64, 128),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_TRIG_RF, 128, 128, 64),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_TRIG_RF, 128, 128, 128),
};
int kNumEntriesBf16Rf = sizeof(kEntriesBf16Rf) / sizeof(kEntriesBf16Rf[0]);
}  // namespace la
