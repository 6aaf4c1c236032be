// Which fold a (dtype, head_dim, GQA group) uses: matrix cores where the
// group makes the page contraction dense enough (bf16, head_dim 128, 4 or 8
// query heads per kv head), vector ALUs otherwise.
#pragma once
#include "fold_mfma.hpp"
#include "fold_valu.hpp"

namespace pkv {

template <typename E, int D, int G> struct FoldFor { using type = ValuFold<E, D, G>; };
template <> struct FoldFor<BF16, 128, 4> { using type = MfmaFold<4>; };
template <> struct FoldFor<BF16, 128, 8> { using type = MfmaFold<8>; };


}  // namespace pkv
