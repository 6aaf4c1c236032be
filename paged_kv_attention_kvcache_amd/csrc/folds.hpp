// Which fold a (dtype, head_dim, GQA group) uses: matrix cores where the
// group makes the page contraction dense enough (bf16, head_dim 128, 4 or 8
// query heads per kv head), vector ALUs otherwise.
#pragma once
#include "fold_mfma.hpp"
#include "fold_valu.hpp"

namespace pkv {

// L: the early-exit variant (each token row read from its own plane's bank).
template <typename E, int D, int G, bool L = false> struct FoldFor {
  using type = ValuFold<E, D, G, L>;
};
template <bool L> struct FoldFor<BF16, 128, 4, L> { using type = MfmaFold<4, false, L>; };
template <bool L> struct FoldFor<BF16, 128, 8, L> { using type = MfmaFold<8, false, L>; };


}  // namespace pkv
