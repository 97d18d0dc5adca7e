// Host build of the library's binary64 -> binary16 conversion (g32.h), for a
// CPU test that compares it with numpy on every binary16 value and midpoint.
#include <stdint.h>

#include "../dequant_gemv_spectra_amd/csrc/g32.h"

extern "C" void convert_batch(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = spectra::f64_to_f16_rne(in[i]);
}
