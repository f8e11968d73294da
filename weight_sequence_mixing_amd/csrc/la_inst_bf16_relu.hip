// Instantiations: bf16 inputs, ReLU feature map (F = d_k).
#include "la_decode.h"
#include "la_forward.h"

namespace la {
#define LA_ENTRY(T, TCODE, PHI, DK, F, DV) \
    {TCODE, PHI, DK, F, DV, plan_chunk<T, PHI>(F), &fwd_launch<T, PHI, DK, F, DV>, &dec_launch<T, PHI, DK, F, DV>}

KernelEntry kEntriesBf16Relu[] = {
    LA_ENTRY(bf16, LA_BF16, LA_PHI_RELU, 64, 64, 64),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_RELU, 64, 64, 128),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_RELU, 128, 128, 64),
    LA_ENTRY(bf16, LA_BF16, LA_PHI_RELU, 128, 128, 128),
};
int kNumEntriesBf16Relu = sizeof(kEntriesBf16Relu) / sizeof(kEntriesBf16Relu[0]);
}  // namespace la
