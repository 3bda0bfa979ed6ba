// odd_f32.hip -- instantiations of the forward and softmax kernels for f32
// rows of an odd length read in aligned pairs (odd.hpp), and of the
// backward's first stage.
#include "odd.hpp"
#include "odd_shapes.hpp"

namespace nf {

#define NF_FWD_ODD(T, VEC, LPR, VPL, TEAMS)                                                        \
    {{LPR, VPL, TEAMS, VEC},                                                                     \
     &launch_fwd_odd<T, LPR, VPL, TEAMS, false, false>,                                           \
     &launch_fwd_odd<T, LPR, VPL, TEAMS, true, false>,                                            \
     &launch_fwd_odd<T, LPR, VPL, TEAMS, false, true>,                                            \
     &launch_fwd_odd<T, LPR, VPL, TEAMS, true, true>},
#define NF_BWD_ODD(T, VEC, LPR, VPL, TEAMS)                                                        \
    {{LPR, VPL, TEAMS, VEC},                                                                     \
     &launch_bwd_odd<T, LPR, VPL, TEAMS, false, false>,                                           \
     &launch_bwd_odd<T, LPR, VPL, TEAMS, true, false>,                                            \
     &launch_bwd_odd<T, LPR, VPL, TEAMS, false, true>,                                            \
     &launch_bwd_odd<T, LPR, VPL, TEAMS, true, true>},
#define NF_SOFTMAX_ODD(T, VEC, LPR, VPL, TEAMS)                                                    \
    {{LPR, VPL, TEAMS, VEC}, &launch_softmax_odd<T, LPR, VPL, TEAMS>},

static const FwdEntry k_fwd[] = {NF_SHAPES_ODD(NF_FWD_ODD, float)};
static const BwdEntry k_bwd[] = {NF_SHAPES_ODD_BWD(NF_BWD_ODD, float)};
static const SoftmaxEntry k_softmax[] = {NF_SHAPES_ODD(NF_SOFTMAX_ODD, float)
                                         NF_SHAPES_ODD_WIDE(NF_SOFTMAX_ODD, float)};

const FwdEntry *fwd_odd_table_f32(int *count) { return table_of(k_fwd, count); }
const BwdEntry *bwd_odd_table_f32(int *count) { return table_of(k_bwd, count); }
const SoftmaxEntry *softmax_odd_table_f32(int *count) { return table_of(k_softmax, count); }

} // namespace nf
