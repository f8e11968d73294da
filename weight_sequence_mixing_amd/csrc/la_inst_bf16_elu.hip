// Instantiations: bf16 inputs, elu+1 feature map (F = d_k).
#include "la_decode.h"
#include "la_forward.h"

namespace la {
#define LA_ENTRY(T, TCODE, PHI, DK, F, DV) \
    {TCODE, PHI, DK, F, DV, plan_chunk<T, PHI>(F), &fwd_launch<T, PHI, DK, F, DV>, &dec_launch<T, PHI, DK, F, DV>}

KernelEntry kEntriesBf16Elu[] = {
    LA_ENTRY(bf16, LA_BF16, LA_PHI_ELU1, 64, 64, 64),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_ELU1, 64, 64, 128),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_ELU1, 128, 128, 64),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_ELU1, 128, 128, 128),
};
int kNumEntriesBf16Elu = sizeof(kEntriesBf16Elu) / sizeof(kEntriesBf16Elu[0]);
}  // namespace la
