// cat_inst_2d_small.hip -- kernel instantiations for one set of transform geometries.
#include "cat_fftconv.hpp"

namespace cat {
const Entry* entries_2d_small(int* n) {
  static const Entry e[] = {
      kern::make_entry<1, 1, false>(),
      kern::make_entry<2, 3, false>(),
      kern::make_entry<3, 4, false>(),
      kern::make_entry<4, 4, false>(),
      kern::make_entry<6, 8, false>(),
      kern::make_entry<8, 8, false>(),
      kern::make_entry<12, 12, false>(),
      kern::make_entry<16, 16, false>(),
      kern::make_entry<32, 32, false>(),
  };
  *n = (int)(sizeof(e) / sizeof(e[0]));
  return e;
}
}  // namespace cat
