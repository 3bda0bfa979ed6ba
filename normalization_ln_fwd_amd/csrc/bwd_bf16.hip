// bwd_bf16.hip -- instantiations of the bwd row kernels for bf16 tensors.
#include "kernels.hpp"
#include "shapes.hpp"

namespace nf {

#define NF_ENTRY(T, VEC, LPR, VPL, TEAMS)                                                          \
    {{LPR, VPL, TEAMS, VEC},                                                                     \
     &launch_bwd<T, VEC, LPR, VPL, TEAMS, false, false>,                                          \
     &launch_bwd<T, VEC, LPR, VPL, TEAMS, true, false>,                                           \
     &launch_bwd<T, VEC, LPR, VPL, TEAMS, false, true>,                                           \
     &launch_bwd<T, VEC, LPR, VPL, TEAMS, true, true>},

static const BwdEntry k_vec[] = {NF_SHAPES_BF16_BWD_VEC(NF_ENTRY)};
static const BwdEntry k_elem[] = {NF_SHAPES_ELEM(NF_ENTRY, bf16)};

const BwdEntry *bwd_table_bf16(bool vectorised, int *count)
{
    *count = vectorised ? int(sizeof k_vec / sizeof k_vec[0]) : int(sizeof k_elem / sizeof k_elem[0]);
    return vectorised ? k_vec : k_elem;
}

} // namespace nf
