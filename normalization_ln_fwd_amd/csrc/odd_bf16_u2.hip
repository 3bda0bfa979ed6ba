// odd_bf16_u2.hip -- the odd-row kernels (odd.hpp) for bf16 rows of N = 2 mod 4:
// 8-byte vectors plus a 2-element unit.
#include "odd.hpp"
#include "odd_shapes.hpp"

namespace nf {

static const FwdEntry k_fwd[] = {NF_SHAPES_ODD_U2_BF16_FWD(NF_FWD_ODD) NF_SHAPES_ODD_U2_WIDE(NF_FWD_ODD, bf16)};
static const BwdEntry k_bwd[] = {NF_SHAPES_ODD_U2_BF16_BWD(NF_BWD_ODD)};
static const SoftmaxEntry k_softmax[] = {NF_SHAPES_ODD_U2_BF16_SOFTMAX(NF_SOFTMAX_ODD) NF_SHAPES_ODD_U2_WIDE(NF_SOFTMAX_ODD, bf16)};

const FwdEntry *fwd_odd_table_bf16_u2(int *count) { return table_of(k_fwd, count); }
const BwdEntry *bwd_odd_table_bf16_u2(int *count) { return table_of(k_bwd, count); }
const SoftmaxEntry *softmax_odd_table_bf16_u2(int *count) { return table_of(k_softmax, count); }

} // namespace nf
