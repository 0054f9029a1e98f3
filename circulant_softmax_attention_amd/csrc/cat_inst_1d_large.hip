// cat_inst_1d_large.hip -- kernel instantiations for one set of transform geometries.
#include "cat_fftconv.hpp"

namespace cat {
const Entry* entries_1d_large(int* n) {
  static const Entry e[] = {
      kern::make_entry<64, 32, true>(),
      kern::make_entry<64, 64, true>(),
  };
  *n = (int)(sizeof(e) / sizeof(e[0]));
  return e;
}
}  // namespace cat
