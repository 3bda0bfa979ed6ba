// odd_f32_u2.hip -- the odd-row kernels (odd.hpp) for fp32 rows of N = 2 mod 4:
// 16-byte vectors plus a 2-element unit (the forward and the backward up to
// 8194 columns).
#include "odd.hpp"
#include "odd_shapes.hpp"

namespace nf {

static const FwdEntry k_fwd[] = {NF_SHAPES_ODD_U2_FWD(NF_FWD_ODD, float)};
static const BwdEntry k_bwd[] = {NF_SHAPES_ODD_U2_F32_BWD(NF_BWD_ODD)};
static const SoftmaxEntry k_softmax[] = {NF_SHAPES_ODD_U2_SOFTMAX(NF_SOFTMAX_ODD, float) NF_SHAPES_ODD_U2_WIDE(NF_SOFTMAX_ODD, float)};

const FwdEntry *fwd_odd_table_f32_u2(int *count) { return table_of(k_fwd, count); }
const BwdEntry *bwd_odd_table_f32_u2(int *count) { return table_of(k_bwd, count); }
const SoftmaxEntry *softmax_odd_table_f32_u2(int *count) { return table_of(k_softmax, count); }

} // namespace nf
