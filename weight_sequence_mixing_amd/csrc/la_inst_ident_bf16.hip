// Instantiations for the random-feature backward (bf16 inputs): the segment-state
// pass and the backward sweeps with the identity feature map, run on phi(q),
// phi(k) computed beforehand (F = 2m plays the role of d_k).
#include "la_backward.h"
#include "la_forward.h"

namespace la {
#define LA_IDENT_ENTRY(F, DV) \
    {LA_BF16, kPhiIdentity, F, F, DV, chunk_len<bf16, kPhiIdentity>(F), &fwd_local_launch<bf16, kPhiIdentity, F, F, DV>, nullptr}
#define LA_IDENT_BWD_ENTRY(F, DV) \
    {LA_BF16, kPhiIdentity, F, F, DV, 32, &bwd_launch<bf16, kPhiIdentity, F, F, DV>, bwd_dlam_fits<bf16, F, F, DV>()}

KernelEntry kEntriesIdentBf16[] = {
    LA_IDENT_ENTRY(64, 64),
    LA_IDENT_ENTRY(64, 128),
    LA_IDENT_ENTRY(128, 64),
    LA_IDENT_ENTRY(128, 128),
    LA_IDENT_ENTRY(256, 64),
    LA_IDENT_ENTRY(256, 128),
};
int kNumEntriesIdentBf16 = sizeof(kEntriesIdentBf16) / sizeof(kEntriesIdentBf16[0]);

BwdEntry kBwdEntriesIdentBf16[] = {
    LA_IDENT_BWD_ENTRY(64, 64),
    LA_IDENT_BWD_ENTRY(64, 128),
    LA_IDENT_BWD_ENTRY(128, 64),
    LA_IDENT_BWD_ENTRY(128, 128),
    LA_IDENT_BWD_ENTRY(256, 64),
    LA_IDENT_BWD_ENTRY(256, 128),
};
int kNumBwdEntriesIdentBf16 = sizeof(kBwdEntriesIdentBf16) / sizeof(kBwdEntriesIdentBf16[0]);
}  // namespace la
