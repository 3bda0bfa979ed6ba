// odd_bf16_u4.hip -- the odd-row kernels (odd.hpp) for bf16 rows of N = 4 mod 8:
// 16-byte vectors plus a 4-element unit.
#include "odd.hpp"
#include "odd_shapes.hpp"

namespace nf {

static const FwdEntry k_fwd[] = {NF_SHAPES_ODD_U4_BF16(NF_FWD_ODD)};
static const BwdEntry k_bwd[] = {NF_SHAPES_ODD_U4_BF16_BWD(NF_BWD_ODD)};
static const SoftmaxEntry k_softmax[] = {NF_SHAPES_ODD_U4_BF16_SOFTMAX(NF_SOFTMAX_ODD)};

const FwdEntry *fwd_odd_table_bf16_u4(int *count) { return table_of(k_fwd, count); }
const BwdEntry *bwd_odd_table_bf16_u4(int *count) { return table_of(k_bwd, count); }
const SoftmaxEntry *softmax_odd_table_bf16_u4(int *count) { return table_of(k_softmax, count); }

} // namespace nf
