// cat_inst_2d_96.hip -- kernel instantiations for one set of transform geometries.
#include "cat_fftconv.hpp"

namespace cat {
const Entry* entries_2d_96(int* n) {
  static const Entry e[] = {
      kern::make_entry<96, 96, false, 2>(),
  };
  *n = (int)(sizeof(e) / sizeof(e[0]));
  return e;
}
}  // namespace cat
