// odd_bf16.hip -- the odd-row kernels (odd.hpp) for bf16 rows of an odd
// length: 4-byte pairs plus one element.
#include "odd.hpp"
#include "odd_shapes.hpp"

namespace nf {

static const FwdEntry k_fwd[] = {NF_SHAPES_ODD_FWD_BF16(NF_FWD_ODD) NF_SHAPES_ODD_WIDE(NF_FWD_ODD, bf16)};
static const BwdEntry k_bwd[] = {NF_SHAPES_ODD_BWD(NF_BWD_ODD, bf16)};
static const SoftmaxEntry k_softmax[] = {NF_SHAPES_ODD_SOFTMAX_BF16(NF_SOFTMAX_ODD) NF_SHAPES_ODD_WIDE(NF_SOFTMAX_ODD, bf16)};

const FwdEntry *fwd_odd_table_bf16_u1(int *count) { return table_of(k_fwd, count); }
const BwdEntry *bwd_odd_table_bf16_u1(int *count) { return table_of(k_bwd, count); }
const SoftmaxEntry *softmax_odd_table_bf16_u1(int *count) { return table_of(k_softmax, count); }

} // namespace nf
