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

static const FwdEntry k_vec[] = {NF_SHAPES_BF16_VEC(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, bf16, 8)};
static const FwdEntry k_elem[] = {NF_SHAPES_ELEM(NF_ENTRY, bf16)};

const FwdEntry *fwd_table_bf16(bool vectorised, int *count)
{
    *count = vectorised ? int(sizeof k_vec / sizeof k_vec[0]) : int(sizeof k_elem / sizeof k_elem[0]);
    return vectorised ? k_vec : k_elem;
}

} // namespace nf
