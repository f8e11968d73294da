// Instantiations for the random-feature backward (fp32 inputs): the segment-state
// pass and the backward sweeps with the identity feature map, run on phi(q),
// phi(k) computed beforehand (F = 2m plays the role of d_k).
#include "la_backward.h"
#include "la_forward.h"

namespace la {
#define LA_IDENT_ENTRY(F, DV) \
    {LA_F32, kPhiIdentity, F, F, DV, chunk_len<float, kPhiIdentity>(F), &fwd_local_launch<float, kPhiIdentity, F, F, DV>, nullptr}
#define LA_IDENT_BWD_ENTRY(F, DV) \
    {LA_F32, kPhiIdentity, F, F, DV, 32, &bwd_launch<float, kPhiIdentity, F, F, DV>, bwd_dlam_fits<float, F, F, DV>()}

KernelEntry kEntriesIdentF32[] = {
    LA_IDENT_ENTRY(64, 64),
    LA_IDENT_ENTRY(64, 128),
    LA_IDENT_ENTRY(128, 64),
    LA_IDENT_ENTRY(128, 128),
};
int kNumEntriesIdentF32 = sizeof(kEntriesIdentF32) / sizeof(kEntriesIdentF32[0]);

BwdEntry kBwdEntriesIdentF32[] = {
    LA_IDENT_BWD_ENTRY(64, 64),
    LA_IDENT_BWD_ENTRY(64, 128),
    LA_IDENT_BWD_ENTRY(128, 64),
    LA_IDENT_BWD_ENTRY(128, 128),
};
int kNumBwdEntriesIdentF32 = sizeof(kBwdEntriesIdentF32) / sizeof(kBwdEntriesIdentF32[0]);
}  // namespace la
