// softmax.hip -- instantiations of the row-softmax kernel for bf16 and fp32.
#include "kernels.hpp"
#include "shapes.hpp"

namespace nf {

#define NF_ENTRY(T, VEC, LPR, VPL, TEAMS) {{LPR, VPL, TEAMS, VEC}, &launch_softmax<T, VEC, LPR, VPL, TEAMS>},

static const SoftmaxEntry k_vec_bf16[] = {NF_SHAPES_BF16_VEC(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, bf16, 8)};
static const SoftmaxEntry k_elem_bf16[] = {NF_SHAPES_ELEM(NF_ENTRY, bf16)};
static const SoftmaxEntry k_vec_f32[] = {NF_SHAPES_F32_VEC(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, float, 4)};
static const SoftmaxEntry k_elem_f32[] = {NF_SHAPES_ELEM(NF_ENTRY, float)};

const SoftmaxEntry *softmax_table_bf16(bool vectorised, int *count)
{
    *count = vectorised ? int(sizeof k_vec_bf16 / sizeof k_vec_bf16[0])
                        : int(sizeof k_elem_bf16 / sizeof k_elem_bf16[0]);
    return vectorised ? k_vec_bf16 : k_elem_bf16;
}

const SoftmaxEntry *softmax_table_f32(bool vectorised, int *count)
{
    *count = vectorised ? int(sizeof k_vec_f32 / sizeof k_vec_f32[0])
                        : int(sizeof k_elem_f32 / sizeof k_elem_f32[0]);
    return vectorised ? k_vec_f32 : k_elem_f32;
}

} // namespace nf
