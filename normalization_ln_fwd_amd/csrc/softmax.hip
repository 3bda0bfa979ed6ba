// softmax.hip -- instantiations of the row-softmax kernel for bf16 and fp32.
#include "kernels.hpp"
#include "shapes.hpp"

namespace nf {

// The 16-byte softmax past the narrow rows: teams of 128 or 256 lanes
// holding two or three vectors each, where the norms take 320-512 lanes
// holding one.  The softmax's two team reductions leave one load per lane
// too little in flight.  Measured on MI355X (us, one-vector teams / these):
// bf16 26214 x 2560 52.2 / 45.0, 21845 x 3072 47.4 / 45.2, 16384 x 4096
// 46.2 / 45.4, 13107 x 5120 47.6 / 46.6; fp32 26214 x 1280 45.6 / 41.1,
// 21845 x 1536 42.8 / 41.4, 10922 x 3072 41.7 / 41.3.
#define NF_SHAPES_SOFTMAX_BF16_VEC(X)                                                            \
    NF_SHAPES_NARROW(X, bf16, 8)                                                                 \
    X(bf16, 8, 64, 5, 4)                                                                         \
    X(bf16, 8, 256, 2, 1)                                                                        \
    X(bf16, 8, 256, 3, 1)                                                                        \
    NF_SHAPES_WIDE_MULTI_VEC(X, bf16, 8)
#define NF_SHAPES_SOFTMAX_F32_VEC(X)                                                             \
    NF_SHAPES_NARROW(X, float, 4)                                                                \
    X(float, 4, 128, 3, 2)                                                                       \
    X(float, 4, 256, 2, 1)                                                                       \
    X(float, 4, 256, 3, 1)                                                                       \
    NF_SHAPES_WIDE_MULTI_VEC(X, float, 4)                                                        \
    X(float, 4, 1024, 4, 1)

#define NF_ENTRY(T, VEC, LPR, VPL, TEAMS) {{LPR, VPL, TEAMS, VEC}, &launch_softmax<T, VEC, LPR, VPL, TEAMS>},

static const SoftmaxEntry k_vec_bf16[] = {NF_SHAPES_SOFTMAX_BF16_VEC(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, bf16, 8)};
static const SoftmaxEntry k_vec4_bf16[] = {NF_SHAPES_BF16_VEC4(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, bf16, 4)};
static const SoftmaxEntry k_vec2_bf16[] = {NF_SHAPES_SHORT_VEC_FINE(NF_ENTRY, bf16, 2)};
static const SoftmaxEntry k_elem_bf16[] = {NF_SHAPES_ELEM(NF_ENTRY, bf16)};
static const SoftmaxEntry k_vec_f32[] = {NF_SHAPES_SOFTMAX_F32_VEC(NF_ENTRY) NF_SHAPES_NARROW_2X(NF_ENTRY, float, 4)};
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
