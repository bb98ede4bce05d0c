// GroupNorm arithmetic shared by the normalising kernel and the conv that normalises its A
// operand on the fly: both include this, so a map normalised either way is bitwise the same.
//
// Corrected asynchronous GroupNorm (DistriFusion summary on atlas.scime.ai, Approach; the
// alternatives are the "Measured effects" table's GroupNorm ablations): the patch normalises
// with the moments of the spliced map, its fresh band moments (m_i, q_i) plus the previous
// step's moments of every other band, each band weighted 1/P; var = E[x^2] - E[x]^2 clamped at 0.
#pragma once

#include <hip/hip_runtime.h>

namespace dp {

// (E, 1/sqrt(var + eps)) of one group from its fresh moments (m, q) and the sums (st_e, st_q) of
// the stale moments the mode combines with them (mode 0 corrected: every band but i; 1 local:
// none; 2 stale: every band).
__device__ __forceinline__ float2 gn_group_norm_params(float m, float q, float st_e, float st_q, int mode, int P,
                                                      float eps) {
    float E = m, Q = q;
    if (mode == 0) {            // corrected: own band fresh, the others stale
        E = (m + st_e) / (float)P;
        Q = (q + st_q) / (float)P;
    } else if (mode == 2) {     // stale: every band from the table
        E = st_e / (float)P;
        Q = st_q / (float)P;
    }
    const float var = fmaxf(Q - E * E, 0.f);
    return make_float2(E, 1.0f / sqrtf(var + eps));
}

// Per-channel affine form of the normalisation: y = x * scale + shift.
__device__ __forceinline__ void gn_scale_shift(float2 er, float gamma, float beta, float& scale, float& shift) {
    scale = er.y * gamma;
    shift = beta - er.x * scale;
}

}  // namespace dp
