// fwd_bf16.hip -- instantiations of the fwd row kernels for bf16 tensors.
#include "kernels.hpp"
#include "shapes.hpp"

namespace nf {

#define NF_ENTRY(T, VEC, LPR, VPL, TEAMS)                                                          \
    {{LPR, VPL, TEAMS, VEC},                                                                     \
     &launch_fwd<T, VEC, LPR, VPL, TEAMS, false, false>,                                          \
     &launch_fwd<T, VEC, LPR, VPL, TEAMS, true, false>,                                           \
     &launch_fwd<T, VEC, LPR, VPL, TEAMS, false, true>,                                           \
     &launch_fwd<T, VEC, LPR, VPL, TEAMS, true, true>},

static const FwdEntry k_vec[] = {NF_SHAPES_FWD_BF16_VEC(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, bf16, 8)};
static const FwdEntry k_vec4[] = {NF_SHAPES_BF16_VEC4_FINE(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, bf16, 4)};
static const FwdEntry k_vec2[] = {NF_SHAPES_SHORT_VEC_FINE(NF_ENTRY, bf16, 2)};
static const FwdEntry k_elem[] = {NF_SHAPES_ELEM(NF_ENTRY, bf16)};

const FwdEntry *fwd_table_bf16(int vec, int *count)
{
    *count = 0;
    switch (vec) {
    case 8: return table_of(k_vec, count);
    case 4: return table_of(k_vec4, count);
    case 2: return table_of(k_vec2, count);
    case 1: return table_of(k_elem, count);
    default: return nullptr;
    }
}

} // namespace nf
