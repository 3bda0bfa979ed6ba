// softmax.hip -- instantiations of the row-softmax kernel for bf16 and fp32.
#include "kernels.hpp"
#include "shapes.hpp"

namespace nf {

#define NF_ENTRY(T, VEC, LPR, VPL, TEAMS) {{LPR, VPL, TEAMS, VEC}, &launch_softmax<T, VEC, LPR, VPL, TEAMS>},

static const SoftmaxEntry k_vec_bf16[] = {NF_SHAPES_BF16_VEC(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, bf16, 8)};
static const SoftmaxEntry k_vec4_bf16[] = {NF_SHAPES_BF16_VEC4(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, bf16, 4)};
static const SoftmaxEntry k_vec2_bf16[] = {NF_SHAPES_SHORT_VEC_FINE(NF_ENTRY, bf16, 2)};
static const SoftmaxEntry k_elem_bf16[] = {NF_SHAPES_ELEM(NF_ENTRY, bf16)};
static const SoftmaxEntry k_vec_f32[] = {NF_SHAPES_F32_VEC(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, float, 4)};
static const SoftmaxEntry k_vec2_f32[] = {NF_SHAPES_SHORT_VEC(NF_ENTRY, float, 2)};
static const SoftmaxEntry k_elem_f32[] = {NF_SHAPES_ELEM(NF_ENTRY, float)};

const SoftmaxEntry *softmax_table_bf16(int vec, int *count)
{
    *count = 0;
    switch (vec) {
    case 8: return table_of(k_vec_bf16, count);
    case 4: return table_of(k_vec4_bf16, count);
    case 2: return table_of(k_vec2_bf16, count);
    case 1: return table_of(k_elem_bf16, count);
    default: return nullptr;
    }
}

const SoftmaxEntry *softmax_table_f32(int vec, int *count)
{
    *count = 0;
    switch (vec) {
    case 4: return table_of(k_vec_f32, count);
    case 2: return table_of(k_vec2_f32, count);
    case 1: return table_of(k_elem_f32, count);
    default: return nullptr;
    }
}

} // namespace nf
