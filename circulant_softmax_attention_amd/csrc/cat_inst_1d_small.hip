// cat_inst_1d_small.hip -- kernel instantiations for one set of transform geometries.
#include "cat_fftconv.hpp"

namespace cat {
const Entry* entries_1d_small(int* n) {
  static const Entry e[] = {
      kern::make_entry<1, 1, true>(),
      kern::make_entry<2, 1, true>(),
      kern::make_entry<2, 2, true>(),
      kern::make_entry<4, 2, true>(),
      kern::make_entry<4, 4, true>(),
      kern::make_entry<8, 4, true>(),
      kern::make_entry<8, 8, true>(),
      kern::make_entry<16, 8, true>(),
      kern::make_entry<16, 16, true>(),
  };
  *n = (int)(sizeof(e) / sizeof(e[0]));
  return e;
}
}  // namespace cat
