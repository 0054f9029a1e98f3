// cat_inst_2d_vit.hip -- kernel instantiations for the patch grids of common
// vision-transformer resolutions: 7 x 7, 14 x 14, 28 x 28 (224 pixels at
// patch 32, 16 and 8), 24 x 24 (384 at 16) and 48 x 48 (768 at 16).
#include "cat_fftconv.hpp"

namespace cat {
const Entry* entries_2d_vit(int* n) {
  static const Entry e[] = {
      kern::make_entry<7, 7, false>(),
      kern::make_entry<14, 14, false>(),
      kern::make_entry<24, 24, false>(),
      kern::make_entry<28, 28, false>(),
      kern::make_entry<48, 48, false, 2>(),
  };
  *n = (int)(sizeof(e) / sizeof(e[0]));
  return e;
}
}  // namespace cat
