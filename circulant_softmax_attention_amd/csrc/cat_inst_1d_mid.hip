// cat_inst_1d_mid.hip -- kernel instantiations for one set of transform geometries.
#include "cat_fftconv.hpp"

namespace cat {
const Entry* entries_1d_mid(int* n) {
  static const Entry e[] = {
      kern::make_entry<32, 16, true>(),
      kern::make_entry<32, 32, true>(),
  };
  *n = (int)(sizeof(e) / sizeof(e[0]));
  return e;
}
}  // namespace cat
