// odd_f32.hip -- the odd-row kernels (odd.hpp) for fp32 rows of an odd
// length: 8-byte pairs plus one element.
#include "odd.hpp"
#include "odd_shapes.hpp"

namespace nf {

static const FwdEntry k_fwd[] = {NF_SHAPES_ODD(NF_FWD_ODD, float)};
static const BwdEntry k_bwd[] = {NF_SHAPES_ODD_BWD(NF_BWD_ODD, float)};
static const SoftmaxEntry k_softmax[] = {NF_SHAPES_ODD(NF_SOFTMAX_ODD, float) NF_SHAPES_ODD_WIDE(NF_SOFTMAX_ODD, float)};

const FwdEntry *fwd_odd_table_f32_u1(int *count) { return table_of(k_fwd, count); }
const BwdEntry *bwd_odd_table_f32_u1(int *count) { return table_of(k_bwd, count); }
const SoftmaxEntry *softmax_odd_table_f32_u1(int *count) { return table_of(k_softmax, count); }

} // namespace nf
